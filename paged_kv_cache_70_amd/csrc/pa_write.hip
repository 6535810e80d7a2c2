// Paged KV-cache write (scatter) for gfx950.
//
// Operation: "P09 · Paged KV 写入 + decode attention" (kuanzhou.online),
// 题面速览 (写) and the write_kv shape trace: for each new token i whose slot is
// non-negative, cache[slot / bs, slot % bs] = k[i] (and v); slot -1 marks a
// padded token and writes nothing.  Because a block's token rows are
// contiguous, slot s is simply row s of the cache viewed as [NB * bs, KVH * D]
// (same page, 细节), so the kernel never splits the slot into (block, offset).
//
// Launch: one thread per 16-byte piece of a token row, K and V handled by the
// same thread; consecutive threads cover consecutive pieces of one row, so
// both the read of k/v and the write into the cache are fully coalesced.
#include "pa_internal.h"

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void write_kv_kernel(
    u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
    const u32x4* __restrict__ k, const u32x4* __restrict__ v,
    const int64_t* __restrict__ slots, uint32_t total_vecs, uint32_t row_vecs,
    int64_t num_slots) {
  const uint32_t idx = blockIdx.x * 256u + threadIdx.x;
  if (idx >= total_vecs) return;
  const uint32_t tok = idx / row_vecs;
  const uint32_t piece = idx - tok * row_vecs;
  const int64_t s = slots[tok];
  // Padding (negative) and out-of-range slots write nothing.
  if (s < 0 || s >= num_slots) return;
  const size_t dst = (size_t)s * row_vecs + piece;
  const u32x4 kv = k[idx];
  const u32x4 vv = v[idx];
  k_cache[dst] = kv;
  v_cache[dst] = vv;
}

hipError_t launch_write_kv(void* k_cache, void* v_cache, const void* k, const void* v,
                           const int64_t* slots, int32_t T, int32_t row_bytes,
                           int64_t num_slots, hipStream_t stream) {
  const uint32_t row_vecs = (uint32_t)row_bytes / 16u;
  const uint64_t total = (uint64_t)T * row_vecs;
  if (total == 0) return hipSuccess;
  const uint32_t grid = (uint32_t)((total + 255u) / 256u);
  hipLaunchKernelGGL(write_kv_kernel, dim3(grid), dim3(256), 0, stream,
                     static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache),
                     static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), slots,
                     (uint32_t)total, row_vecs, num_slots);
  return hipGetLastError();
}

}  // namespace pa
