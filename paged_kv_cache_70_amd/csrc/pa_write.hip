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
// 16 bytes, V [NB, KVH, D, bs].  Row r = h * D + d of (block, head) holds one
// element per token slot, so consecutive slots of a block are adjacent
// elements of a row (and, for K, adjacent 16-byte groups).
//
// A workgroup takes 16 new tokens and 32 of their 16-byte groups.  K stores
// run with the token as the fastest lane index: when the 16 tokens occupy
// consecutive slots (any prefill chunk, whatever its offset in the block),
// each K group becomes one 256-byte run.  V is first staged in LDS with
// coalesced 16-byte reads, then read back transposed; runs of 16 bytes of
// tokens (8 bf16, 4 fp32) in consecutive slots of one block, aligned, are
// stored as one 16-byte store per V row.  A workgroup with no such run (a
// decode step's tokens, one per sequence) stores V element by element with
// the token as the fastest lane index.
constexpr int kWTok = 16;        // tokens per workgroup
constexpr int kWGrp = 32;        // 16-byte groups per workgroup
constexpr int kWRow = kWGrp * 16 + 16;   // LDS bytes per token row (16 bytes of padding)

template <typename E>
__global__ __launch_bounds__(256) void write_kv_vllm_kernel(
    u32x4* __restrict__ k_cache, E* __restrict__ v_cache,
    const u32x4* __restrict__ k, const u32x4* __restrict__ v,
    const int64_t* __restrict__ slots, uint32_t num_tokens, uint32_t row_groups,
    int32_t bs_log2, int64_t num_slots) {
  constexpr uint32_t X = 16 / sizeof(E);
  __shared__ __attribute__((aligned(16))) unsigned char tile[kWTok * kWRow];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t t0 = blockIdx.x * kWTok;
  const uint32_t g0 = blockIdx.y * kWGrp;

  // Every load is issued before the first barrier: this lane's slot (token
  // i = lane mod 16), V's 16-byte pieces for the LDS stage, then the K groups
  // this lane stores, which wait only for the slot.  For a few tokens (a
  // decode step) the kernel is latency-bound, and the V and K loads overlap.
  const uint32_t i = lane & (kWTok - 1);
  int64_t s = (t0 + i < num_tokens) ? slots[t0 + i] : -1;
  constexpr uint32_t NV = kWTok * kWGrp / 256;
  u32x4 vreg[NV];
#pragma unroll
  for (uint32_t j = 0; j < NV; ++j) {
    const uint32_t idx = tid + 256u * j, ti = idx / kWGrp, q = idx % kWGrp;
    vreg[j] = u32x4{0u, 0u, 0u, 0u};
    if (t0 + ti < num_tokens && g0 + q < row_groups)
      vreg[j] = __builtin_nontemporal_load(&v[(size_t)(t0 + ti) * row_groups + g0 + q]);
  }
  s = (s >= 0 && s < num_slots) ? s : -1;   // invalid slots and tokens past the end store nothing
  const bool live = s >= 0;
  const size_t blk = live ? (size_t)(s >> bs_log2) : 0;
  const size_t off = live ? (size_t)(s & ((1 << bs_log2) - 1)) : 0;
  // K: lane (token i, group q); one 16-byte load and store per group.
  constexpr uint32_t NK = kWGrp / 16;
  u32x4 kreg[NK];
#pragma unroll
  for (uint32_t j = 0; j < NK; ++j) {
    const uint32_t q = (lane >> 4) + 4u * wave + 16u * j;
    kreg[j] = u32x4{0u, 0u, 0u, 0u};
    if (live && g0 + q < row_groups) kreg[j] = __builtin_nontemporal_load(&k[(size_t)(t0 + i) * row_groups + g0 + q]);
  }

  // Stage V: 16 rows of up to 32 groups, 32 consecutive threads per token row.
#pragma unroll
  for (uint32_t j = 0; j < NV; ++j) {
    const uint32_t idx = tid + 256u * j, ti = idx / kWGrp, q = idx % kWGrp;
    *reinterpret_cast<u32x4*>(tile + ti * kWRow + q * 16) = vreg[j];
  }

  // Runs: GT = 16 bytes / element consecutive tokens that fill GT
  // consecutive slots of one block starting at a multiple of GT (then one
  // 16-byte store covers the run in every V row).  Every wave holds the 16
  // slots in lanes 0-15, so a ballot of "this token continues its run" gives
  // the run flags, the same in every wave.
  constexpr uint32_t GT = X;                 // tokens per 16-byte V run
  constexpr uint32_t NRUN = kWTok / GT;
  constexpr uint64_t kRunBits = (1ull << GT) - 1;
  const int64_t prev = __shfl_up(s, 1u);
  const bool starts = (i & (GT - 1)) == 0;
  const bool link = starts ? (live && (s & (GT - 1)) == 0 && (off + GT) <= (1u << bs_log2))
                           : (live && prev >= 0 && s == prev + 1);
  const uint64_t links = __ballot(link);
  bool any_run = false;
#pragma unroll
  for (uint32_t r = 0; r < NRUN; ++r) any_run |= ((links >> (r * GT)) & kRunBits) == kRunBits;

  // Threads 0-15 are lanes 0-15 of wave 0: token tid.
  __shared__ int64_t s_slot[kWTok];
  if (tid < kWTok) s_slot[tid] = s;

#pragma unroll
  for (uint32_t j = 0; j < NK; ++j) {
    const uint32_t q = (lane >> 4) + 4u * wave + 16u * j;
    if (live && g0 + q < row_groups) k_cache[((blk * row_groups + g0 + q) << bs_log2) + off] = kreg[j];
  }
  __syncthreads();

  const uint32_t elems = min((uint32_t)kWGrp, row_groups - g0) * X;
  const size_t row0 = (size_t)g0 * X;
  const size_t rows = (size_t)row_groups * X;

  // V without runs (the decode step's one token per sequence): lane (token i,
  // element e), four adjacent rows of one token per wave store, block and
  // offset computed once per lane.
  if (!any_run) {
    const E* trow = reinterpret_cast<const E*>(tile + i * kWRow);
#pragma unroll 4
    for (uint32_t e = (lane >> 4) + 4u * wave; e < kWGrp * X; e += 16u) {
      if (live && e < elems) v_cache[((blk * rows + row0 + e) << bs_log2) + off] = trow[e];
    }
    return;
  }

  // V with runs: thread (element e of the slice, run r of GT tokens).  A run
  // of consecutive aligned slots is one 16-byte store of its GT elements of
  // row e (gathered from the staged rows); otherwise each live token of the
  // run stores its own element.  The padded LDS row stride puts the tokens of
  // a run on distinct banks.
  for (uint32_t w = tid; w < kWGrp * X * NRUN; w += 256u) {
    const uint32_t e = w / NRUN, r = w % NRUN;
    if (e >= elems) continue;
    E vals[GT];
#pragma unroll
    for (uint32_t j = 0; j < GT; ++j) vals[j] = reinterpret_cast<const E*>(tile + (r * GT + j) * kWRow)[e];
    if (((links >> (r * GT)) & kRunBits) == kRunBits) {
      const int64_t first = s_slot[r * GT];
      const size_t b0 = (size_t)(first >> bs_log2), o0 = (size_t)(first & ((1 << bs_log2) - 1));
      u32x4 pk;
      __builtin_memcpy(&pk, vals, 16);
      *reinterpret_cast<u32x4*>(v_cache + ((b0 * rows + row0 + e) << bs_log2) + o0) = pk;
    } else {
#pragma unroll
      for (uint32_t j = 0; j < GT; ++j) {
        const int64_t sj = s_slot[r * GT + j];
        if (sj >= 0)
          v_cache[(((size_t)(sj >> bs_log2) * rows + row0 + e) << bs_log2) + (size_t)(sj & ((1 << bs_log2) - 1))] =
              vals[j];
      }
    }
  }
}

hipError_t launch_write_kv_vllm(void* k_cache, void* v_cache, const void* k, const void* v,
                                const int64_t* slots, int32_t T, int32_t row_bytes, int32_t elem_bytes,
                                int32_t bs_log2, int64_t num_slots, hipStream_t stream) {
  const uint32_t row_groups = (uint32_t)row_bytes / 16u;
  if (T <= 0 || row_groups == 0) return hipSuccess;
  const dim3 grid((uint32_t)((T + kWTok - 1) / kWTok), (row_groups + kWGrp - 1) / kWGrp);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(write_kv_vllm_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       static_cast<u32x4*>(k_cache), static_cast<uint16_t*>(v_cache),
                       static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), slots,
                       (uint32_t)T, row_groups, bs_log2, num_slots);
  else
    hipLaunchKernelGGL(write_kv_vllm_kernel<uint32_t>, grid, dim3(256), 0, stream,
                       static_cast<u32x4*>(k_cache), static_cast<uint32_t*>(v_cache),
                       static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), slots,
                       (uint32_t)T, row_groups, bs_log2, num_slots);
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
