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

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
  const u32x4 kv = k_new[i];
  const u32x4 vv = v_new[i];
  k_cache[slot * chunks_per_row + c] = kv;
  v_cache[slot * chunks_per_row + c] = vv;
}

}  // namespace

int launch_kv_write(const KvWriteArgs& a) {
  const int chunks_per_row = a.num_kv_heads * a.head_dim / 8;  // 16-byte chunks
  const long long total = (long long)a.num_tokens * chunks_per_row;
  const long long num_slots = (long long)a.num_pages * a.page_size;
  const unsigned grid = (unsigned)((total + kWriteThreads - 1) / kWriteThreads);
  void* args[] = {(void*)&a.k_new,   (void*)&a.v_new,   (void*)&a.slot_mapping,
                  (void*)&a.k_cache, (void*)&a.v_cache, (void*)&total,
                  (void*)&chunks_per_row, (void*)&num_slots};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&kv_write_kernel), dim3(grid),
                              dim3(kWriteThreads), args, 0,
                              reinterpret_cast<hipStream_t>(a.stream));
}

}  // namespace pa
