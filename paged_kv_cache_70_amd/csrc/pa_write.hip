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
  // The new rows are read once: non-temporal loads keep them from displacing
  // cache lines (7% faster at 65,536 tokens).  The stores stay ordinary:
  // non-temporal stores measured 16% slower.
  const u32x4 kv = __builtin_nontemporal_load(&k[idx]);
  const u32x4 vv = __builtin_nontemporal_load(&v[idx]);
  k_cache[dst] = kv;
  v_cache[dst] = vv;
}

// The same scatter into vLLM's cache layout ("PagedAttention kernel：paged KV
// cache 与 block table", 深入原理): K [NB, KVH, D/x, bs, x] with x elements =
// 16 bytes, V [NB, KVH, D, bs].  One thread per 16-byte group of x elements
// (token, kv head, group g): the K group is one 16-byte store at
// (block, head, g, offset); its x V elements go to x rows d = g x + e of
// (block, head), each at column `offset` (stride bs elements).
template <typename E>
__global__ __launch_bounds__(256) void write_kv_vllm_kernel(
    u32x4* __restrict__ k_cache, E* __restrict__ v_cache,
    const u32x4* __restrict__ k, const E* __restrict__ v,
    const int64_t* __restrict__ slots, uint32_t total_groups, uint32_t row_groups,
    int32_t bs_log2, int64_t num_slots) {
  constexpr uint32_t X = 16 / sizeof(E);
  const uint32_t idx = blockIdx.x * 256u + threadIdx.x;
  if (idx >= total_groups) return;
  const uint32_t tok = idx / row_groups;
  const uint32_t rem = idx - tok * row_groups;     // kv head * (D / x) + group
  const int64_t s = slots[tok];
  if (s < 0 || s >= num_slots) return;
  const size_t blk = (size_t)(s >> bs_log2);
  const size_t off = (size_t)(s & ((1 << bs_log2) - 1));
  const size_t col = (blk * row_groups + rem) << bs_log2;   // (block, head, group) row of bs columns
  k_cache[col + off] = k[idx];
  const E* src = v + (size_t)idx * X;
#pragma unroll
  for (uint32_t e = 0; e < X; ++e) v_cache[((col * X) + ((size_t)e << bs_log2)) + off] = src[e];
}

hipError_t launch_write_kv_vllm(void* k_cache, void* v_cache, const void* k, const void* v,
                                const int64_t* slots, int32_t T, int32_t row_bytes, int32_t elem_bytes,
                                int32_t bs_log2, int64_t num_slots, hipStream_t stream) {
  const uint32_t row_groups = (uint32_t)row_bytes / 16u;
  const uint64_t total = (uint64_t)T * row_groups;
  if (total == 0) return hipSuccess;
  const uint32_t grid = (uint32_t)((total + 255u) / 256u);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(write_kv_vllm_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream,
                       static_cast<u32x4*>(k_cache), static_cast<uint16_t*>(v_cache),
                       static_cast<const u32x4*>(k), static_cast<const uint16_t*>(v), slots,
                       (uint32_t)total, row_groups, bs_log2, num_slots);
  else
    hipLaunchKernelGGL(write_kv_vllm_kernel<uint32_t>, dim3(grid), dim3(256), 0, stream,
                       static_cast<u32x4*>(k_cache), static_cast<uint32_t*>(v_cache),
                       static_cast<const u32x4*>(k), static_cast<const uint32_t*>(v), slots,
                       (uint32_t)total, row_groups, bs_log2, num_slots);
  return hipGetLastError();
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
