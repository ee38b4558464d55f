// Device helpers shared by the decode, multi-query and merge kernels: BF16 and
// FP8 conversions, the register software pipeline and the log-sum-exp merge of
// split partials. Included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// BF16 -> FP32 is exact: the BF16 bits are the high half of the FP32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// FP32 -> BF16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// FP8 E4M3 (OCP) -> FP32 for the 4 codes of a word, with gfx950's
// v_cvt_pk_f32_fp8 (exact: every E4M3 value is an FP32 value).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* f) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  f[0] = lo.x;
  f[1] = lo.y;
  f[2] = hi.x;
  f[3] = hi.y;
}

// 8 FP8 codes (2 words) -> 8 BF16 values packed for an MFMA operand. Exact:
// E4M3 values have 3 mantissa bits and exponents within BF16's range, so the
// FP32 value's upper half is the BF16 value.
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  float f[8];
  fp8x4_to_f32(w0, f);
  fp8x4_to_f32(w1, f + 4);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = (__float_as_uint(f[2 * i]) >> 16) | (__float_as_uint(f[2 * i + 1]) & 0xffff0000u);
  return r;
}

// FP8 E4M3 ("FN") codes of four FP32 values, byte j from y[j]: saturated to
// +-448 (the format has no infinity), rounded to nearest even by gfx950's
// v_cvt_pk_fp8_f32, NaN stored as 0x7F. The explicit clamp makes the
// conversion's own overflow handling irrelevant; NaN is set after it.
__device__ __forceinline__ uint32_t e4m3x4(const float* y) {
  float c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = __builtin_fminf(__builtin_fmaxf(y[j], -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  uint32_t u = (uint32_t)w;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (__builtin_isnan(y[j])) u = (u & ~(0xFFu << (8 * j))) | (0x7Fu << (8 * j));
  return u;
}

// The same encoding for two values: codes in bits 0-7 (a) and 8-15 (b).
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  const float ca = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
  const float cb = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
  uint32_t u = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
  if (__builtin_isnan(a)) u = (u & ~0xFFu) | 0x7Fu;
  if (__builtin_isnan(b)) u = (u & ~0xFF00u) | 0x7F00u;
  return u;
}

// Eight BF16 values (one 16-byte chunk) divided by `scale` (IEEE FP32
// division) and encoded: the 8 codes of the chunk, in order.
__device__ __forceinline__ u32x2 bf16x8_to_e4m3(u32x4 x, float scale) {
  float y[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    y[2 * j] = bf16_lo(x[j]) / scale;
    y[2 * j + 1] = bf16_hi(x[j]) / scale;
  }
  u32x2 r;
  r[0] = e4m3x4(y);
  r[1] = e4m3x4(y + 4);
  return r;
}

// Software pipeline over n items held in NB register slots (item i in slot
// i % NB): items i+1 .. i+NB-1 are loading while item i is used. In the steady
// state every prefetch is issued unconditionally and pinned before the use
// with a scheduling barrier, so the compiler's wait counts let exactly the
// consumed item's loads complete; the tail (< 2*NB-1 items) guards each one.
// `load(item, slot)` and `use(item, slot)` receive compile-time slot indices
// after unrolling.
//
// On the path into the steady-state loop the first NB-1 loads are issued
// unconditionally: if some path could enter the loop with fewer loads in
// flight, the compiler would have to assume the youngest loads are the ones
// being used and wait for all of them, collapsing the pipeline to depth 1.
// `ready` runs once after the first NB-1 loads are issued and before the
// first use: work the uses depend on overlaps those loads' latency.
template <int NB, class Load, class Use, class Ready>
__device__ __forceinline__ void pipeline(int n, Load&& load, Use&& use, Ready&& ready) {
  int j = 0;
  if (n > 2 * NB - 2) {
#pragma unroll
    for (int i = 0; i < NB - 1; ++i) load(i, i);
    ready();
    for (; j + 2 * NB - 2 < n; j += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        load(j + u + NB - 1, (u + NB - 1) % NB);
        __builtin_amdgcn_sched_barrier(0);
        use(j + u, u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NB - 1; ++i)
      if (i < n) load(i, i);
    ready();
  }
#pragma unroll
  for (int u = 0; u < 2 * NB - 2; ++u) {
    if (j + u < n) {
      if (j + u + NB - 1 < n) load(j + u + NB - 1, (u + NB - 1) % NB);
      use(j + u, u % NB);
    }
  }
}

template <int NB, class Load, class Use>
__device__ __forceinline__ void pipeline(int n, Load&& load, Use&& use) {
  pipeline<NB>(n, load, use, [] {});
}

// Log-sum-exp merge of the first nv split partials of one (sequence, query
// head) row, for the 4 dims d4 .. d4+3: M = max m_s, out = sum 2^(m_s-M) acc_s
// / sum 2^(m_s-M) l_s. The partials of up to C splits are loaded together,
// then folded into a running state, so a row costs one memory round trip per
// C splits. nv == 0 (empty context) gives zeros.
constexpr int kMergeChunk = 8;

struct MergeState {
  float m = -INFINITY;  // running max of the folded m_s
  float den = 0.f;      // sum 2^(m_s - m) l_s
  f32x4 num = {0.f, 0.f, 0.f, 0.f};  // sum 2^(m_s - m) acc_s
};

// Fold the first `count` (<= C) loaded partials into the state.
template <int C>
__device__ __forceinline__ void merge_fold(MergeState& st, const float2 (&mlv)[C],
                                           const f32x4 (&av)[C], int count) {
  float mc = st.m;
#pragma unroll
  for (int i = 0; i < C; ++i)
    if (i < count) mc = fmaxf(mc, mlv[i].x);
  const float a = st.m == -INFINITY ? 0.f : fast_exp2(st.m - mc);
  st.den *= a;
  st.num *= a;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    if (i < count) {
      const float w = fast_exp2(mlv[i].x - mc);
      st.den = fmaf(w, mlv[i].y, st.den);
#pragma unroll
      for (int e = 0; e < 4; ++e) st.num[e] = fmaf(w, av[i][e], st.num[e]);
    }
  }
  st.m = mc;
}

// Load the partials of splits s0 .. s0 + min(count, C) - 1.
template <int D, int C>
__device__ __forceinline__ void merge_load(const float* ml, const float* acc, int s0, int count,
                                           float2 (&mlv)[C], f32x4 (&av)[C]) {
#pragma unroll
  for (int i = 0; i < C; ++i) {
    if (i < count) {
      mlv[i] = *reinterpret_cast<const float2*>(ml + 2 * (s0 + i));
      av[i] = *reinterpret_cast<const f32x4*>(acc + (size_t)(s0 + i) * D);
    }
  }
}

__device__ __forceinline__ f32x4 merge_result(const MergeState& st, int nv) {
  f32x4 res = {0.f, 0.f, 0.f, 0.f};
  if (nv > 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) res[e] = st.num[e] / st.den;
  }
  return res;
}

__device__ __forceinline__ void store_bf16x4(uint16_t* dst, f32x4 v) {
  uint2 packed;
  packed.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  packed.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<uint2*>(dst) = packed;
}

}  // namespace
}  // namespace pa
