// Attention prologue for gfx950 (MI355X): per-head RMSNorm of q and k (QK-norm),
// NeoX RoPE at each token's position, and the paged KV write, in one kernel.
//
// "Qwen 3" (TensorSharp docs), section 3 "Forward graph" and section 4.1
// "Attention": after the QKV projection every query and key head is normalised
// on its own (RMSNorm, head_dim weights), rotated NeoX-style (dim i pairs with
// dim i + D/2), and K and V are appended to the cache; "Qwen3-14B" (pypto-lib
// models page), section "decode_fwd", runs this as the attention kernel's
// phase 0. Per head vector x, weight w, position p:
//   y = x / sqrt(mean(x^2) + eps) * w
//   theta_i = p * base^(-2i/D) / scale
//   out_i = y_i cos theta_i - y_{i+D/2} sin theta_i
//   out_{i+D/2} = y_{i+D/2} cos theta_i + y_i sin theta_i
// V is written as given; K after norm and RoPE; q goes to q_out (the attention
// call applies the logit scale).
//
// One 256-thread workgroup per token. The D/2 rotation angles of the token are
// computed once in FP64 (exact for any position a page table can address, then
// rounded to FP32 cos/sin) and shared through LDS. Every head row of the token
// (Hq q rows, Hkv k rows, Hkv v rows) is handled by D/8 lanes holding 8
// consecutive dims each (one 16-byte load): the sum of squares is a lane
// butterfly (same value and order on every lane), and the RoPE partner values
// come from the lane D/16 away by a shuffle. HBM-bound: every byte is read once
// and written once.
//
// kFp8: the pools hold FP8 E4M3 codes with one FP32 scale each. The K row is
// first rounded to BF16 exactly as for BF16 pools, then each value is divided
// by k_scale and encoded (saturating, nearest even), as pa_kv_write_fp8 stores
// a BF16 row; V is encoded from its BF16 input with v_scale. The result is
// the BF16 prologue followed by the FP8 KV write, in one pass.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace pa {
namespace {

constexpr int kProThreads = 256;

template <int D, bool kFp8>
__global__ __launch_bounds__(kProThreads) void prologue_kernel(
    const uint16_t* q_in, const uint16_t* __restrict__ k_in,
    const uint16_t* __restrict__ v_in, const uint16_t* __restrict__ q_norm_w,
    const uint16_t* __restrict__ k_norm_w, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ slot_mapping, uint16_t* q_out, void* __restrict__ k_cache,
    void* __restrict__ v_cache, int num_q_heads, int num_kv_heads, long long num_slots,
    float eps, double log2_base, double inv_scale, float k_scale, float v_scale) {
  constexpr int LPR = D / 8;              // lanes per head row
  constexpr int RPP = kProThreads / LPR;  // rows per pass
  constexpr int H = D / 2;
  __shared__ float s_cos[H];
  __shared__ float s_sin[H];
  // 8 BF16 values at element offset e of a pool: copied, or encoded to FP8
  auto store_row_chunk = [](void* pool, size_t e, u32x4 x, float scale) {
    if constexpr (kFp8)
      *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(pool) + e) = bf16x8_to_e4m3(x, scale);
    else
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(pool) + e) = x;
  };

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < H) {
    const double inv_freq = exp2(-(2.0 * tid / D) * log2_base) * inv_scale;
    const double th = (double)positions[t] * inv_freq;
    double s, c;
    sincos(th, &s, &c);
    s_cos[tid] = (float)c;
    s_sin[tid] = (float)s;
  }
  const long long slot = slot_mapping[t];
  const bool write_kv = slot >= 0 && slot < num_slots;
  // [page, token, kv_head, dim] pools: slot p*P + i is row slot*Hkv + h of the pool
  const size_t kv_row = write_kv ? (size_t)slot * num_kv_heads : 0;
  __syncthreads();

  const int c = tid % LPR;     // dims 8c .. 8c+7
  const int rr = tid / LPR;    // row within the pass
  const int rows = num_q_heads + 2 * num_kv_heads;
  const float inv_d = 1.0f / D;
  for (int r = rr; r < rows; r += RPP) {  // uniform trip count per row group
    const bool is_q = r < num_q_heads;
    const bool is_k = !is_q && r < num_q_heads + num_kv_heads;
    const int h = is_q ? r : (is_k ? r - num_q_heads : r - num_q_heads - num_kv_heads);
    const uint16_t* src = is_q ? q_in + ((size_t)t * num_q_heads + h) * D
                               : (is_k ? k_in : v_in) + ((size_t)t * num_kv_heads + h) * D;
    const u32x4 xw = load16(src + 8 * c);
    if (!is_q && !is_k) {  // V: a plain copy (or its codes) into its slot
      if (write_kv) store_row_chunk(v_cache, (kv_row + h) * D + 8 * c, xw, v_scale);
      continue;
    }
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(xw[i]);
      x[2 * i + 1] = bf16_hi(xw[i]);
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) ss += __shfl_xor(ss, off);
    const float rinv = 1.0f / sqrtf(ss * inv_d + eps);
    const u32x4 ww = load16((is_q ? q_norm_w : k_norm_w) + 8 * c);
    float y[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[2 * i] = x[2 * i] * rinv * bf16_lo(ww[i]);
      y[2 * i + 1] = x[2 * i + 1] * rinv * bf16_hi(ww[i]);
    }
    // partner dims (d + D/2 or d - D/2) live in the lane LPR/2 away
    const bool first = c < LPR / 2;
    const int f0 = (first ? 8 * c : 8 * c - H);  // frequency index of y[0]
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float partner = __shfl_xor(y[i], LPR / 2);
      const float cs = s_cos[f0 + i];
      const float sn = s_sin[f0 + i];
      o[i] = first ? y[i] * cs - partner * sn : y[i] * cs + partner * sn;
    }
    u32x4 ow;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ow[i] = (uint32_t)f32_to_bf16(o[2 * i]) | ((uint32_t)f32_to_bf16(o[2 * i + 1]) << 16);
    if (is_q) {
      *reinterpret_cast<u32x4*>(q_out + ((size_t)t * num_q_heads + h) * D + 8 * c) = ow;
    } else if (write_kv) {
      store_row_chunk(k_cache, (kv_row + h) * D + 8 * c, ow, k_scale);
    }
  }
}

template <int D, bool kFp8>
int launch_prologue_d(const PrologueArgs& a) {
  hipStream_t stream = reinterpret_cast<hipStream_t>(a.stream);
  const long long num_slots = (long long)a.num_pages * a.page_size;
  const double log2_base = log2((double)a.rope_base);
  const double inv_scale = 1.0 / (double)a.rope_scale;
  void* args[] = {(void*)&a.q_in,       (void*)&a.k_in,        (void*)&a.v_in,
                  (void*)&a.q_norm_w,   (void*)&a.k_norm_w,    (void*)&a.positions,
                  (void*)&a.slot_mapping, (void*)&a.q_out,     (void*)&a.k_cache,
                  (void*)&a.v_cache,    (void*)&a.num_q_heads, (void*)&a.num_kv_heads,
                  (void*)&num_slots,    (void*)&a.eps,
                  (void*)&log2_base,    (void*)&inv_scale, (void*)&a.k_scale,
                  (void*)&a.v_scale};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&prologue_kernel<D, kFp8>),
                              dim3(a.num_tokens), dim3(kProThreads), args, 0, stream);
}

}  // namespace

int launch_prologue(const PrologueArgs& a) {
  if (a.fp8) return a.head_dim == 128 ? launch_prologue_d<128, true>(a) : launch_prologue_d<256, true>(a);
  return a.head_dim == 128 ? launch_prologue_d<128, false>(a) : launch_prologue_d<256, false>(a);
}

}  // namespace pa
