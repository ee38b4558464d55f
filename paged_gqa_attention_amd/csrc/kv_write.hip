// Paged KV write for gfx950: scatter a step's new K/V rows into the pools.
//
// "Qwen 3" (TensorSharp docs), section 11 "Batched / paged forward": each
// token's K and V are written at block_id * block_size + offset of the layer's
// paged buffer, the flat slot that slot_mapping holds. In the
// [page, token, kv_head, dim] pool the Hkv*D values of one token are
// contiguous, so slot s owns bytes [s * row_bytes, (s+1) * row_bytes) and the
// write is a row copy. Every thread copies one 16-byte chunk of K and the same
// chunk of V; a negative slot (padding) or a slot past the pool writes nothing.
// HBM-bound: per token 2 rows read and 2 rows written.
//
// FP8 pools (one byte per value, E4M3 "FN" encoding, one FP32 scale per pool):
// each BF16 value x is stored as the code of x / scale, the quotient taken in
// FP32 with IEEE division, saturated to +-448 (the format has no infinity),
// rounded to nearest even by v_cvt_pk_fp8_f32; NaN is stored as 0x7F. The
// decode and multi-query kernels read code * scale back, so the cache keeps
// the fp8_e4m3 KV dtype the orcarouter page measures against NVFP4 KV.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace pa {
namespace {


constexpr int kWriteThreads = 256;

__global__ __launch_bounds__(kWriteThreads) void kv_write_kernel(
    const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
    const int32_t* __restrict__ slot_mapping, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, long long total_chunks, int chunks_per_row, long long num_slots) {
  const long long i = (long long)blockIdx.x * kWriteThreads + threadIdx.x;
  if (i >= total_chunks) return;
  const long long t = i / chunks_per_row;
  const int c = (int)(i - t * chunks_per_row);
  const long long slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // padding token / outside the pool
  // nothing reads these lines again in this kernel: non-temporal loads and
  // stores (measured on MI355X: 65,536 rows 103.5 -> 100.4 us)
  const u32x4 kv = __builtin_nontemporal_load(k_new + i);
  const u32x4 vv = __builtin_nontemporal_load(v_new + i);
  __builtin_nontemporal_store(kv, k_cache + slot * chunks_per_row + c);
  __builtin_nontemporal_store(vv, v_cache + slot * chunks_per_row + c);
}

__global__ __launch_bounds__(kWriteThreads) void kv_write_fp8_kernel(
    const u32x4* __restrict__ k_new, const u32x4* __restrict__ v_new,
    const int32_t* __restrict__ slot_mapping, u32x2* __restrict__ k_codes,
    u32x2* __restrict__ v_codes, long long total_chunks, int chunks_per_row, long long num_slots,
    float k_scale, float v_scale) {
  const long long i = (long long)blockIdx.x * kWriteThreads + threadIdx.x;
  if (i >= total_chunks) return;
  const long long t = i / chunks_per_row;
  const int c = (int)(i - t * chunks_per_row);
  const long long slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;  // padding token / outside the pool
  const u32x4 kv = k_new[i];
  const u32x4 vv = v_new[i];
  k_codes[slot * chunks_per_row + c] = bf16x8_to_e4m3(kv, k_scale);
  v_codes[slot * chunks_per_row + c] = bf16x8_to_e4m3(vv, v_scale);
}

}  // namespace

int launch_kv_write(const KvWriteArgs& a) {
  const int chunks_per_row = a.num_kv_heads * a.head_dim / 8;  // 16-byte chunks
  const long long total = (long long)a.num_tokens * chunks_per_row;
  const long long num_slots = (long long)a.num_pages * a.page_size;
  const unsigned grid = (unsigned)((total + kWriteThreads - 1) / kWriteThreads);
  if (a.fp8) {
    void* args[] = {(void*)&a.k_new,   (void*)&a.v_new,   (void*)&a.slot_mapping,
                    (void*)&a.k_cache, (void*)&a.v_cache, (void*)&total,
                    (void*)&chunks_per_row, (void*)&num_slots, (void*)&a.k_scale,
                    (void*)&a.v_scale};
    return (int)hipLaunchKernel(reinterpret_cast<const void*>(&kv_write_fp8_kernel), dim3(grid),
                                dim3(kWriteThreads), args, 0,
                                reinterpret_cast<hipStream_t>(a.stream));
  }
  void* args[] = {(void*)&a.k_new,   (void*)&a.v_new,   (void*)&a.slot_mapping,
                  (void*)&a.k_cache, (void*)&a.v_cache, (void*)&total,
                  (void*)&chunks_per_row, (void*)&num_slots};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&kv_write_kernel), dim3(grid),
                              dim3(kWriteThreads), args, 0,
                              reinterpret_cast<hipStream_t>(a.stream));
}

}  // namespace pa
