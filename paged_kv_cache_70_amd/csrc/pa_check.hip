// Checked mode: kernels that test the device-side preconditions of the write,
// the decode and the prefill and report every kind of violation as a bit of a
// caller-owned error word.  "P09 · Paged KV 写入 + decode attention" shows
// what happens without them: a -1 slot taken as an index overwrites the last
// row with no error (直觉与类比), and a garbage table entry gives an index
// error or silently wrong K/V (易错点).  The hot-path kernels stay
// memory-safe on such inputs but say nothing; these kernels say what broke.
//
// Flags are set with vector atomics (global_atomic_or), only by the lanes that
// find a violation.  The kernels read what the hot path reads (table entries
// below ceil(n / bs), the slots, the lengths), nothing else.
#include "../../include/paged_kv.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kCheckThreads = 256;

__device__ __forceinline__ void flag(uint32_t* err, uint32_t bit) { atomicOr(err, bit); }

// Zeroes the slot bitmap (a fill kernel: no memset node in a captured graph).
__global__ __launch_bounds__(kCheckThreads) void clear_words_kernel(uint32_t* __restrict__ w, uint32_t n) {
  for (uint32_t i = blockIdx.x * kCheckThreads + threadIdx.x; i < n; i += gridDim.x * kCheckThreads) w[i] = 0u;
}

// One thread per token: a valid slot past the pool, or a slot already marked
// in the bitmap by another token.
__global__ __launch_bounds__(kCheckThreads) void check_slots_kernel(const int64_t* __restrict__ slots, int32_t T,
                                                                    int64_t num_slots, uint32_t* __restrict__ bitmap,
                                                                    uint32_t* __restrict__ err) {
  const int i = blockIdx.x * kCheckThreads + threadIdx.x;
  if (i >= T) return;
  const int64_t s = slots[i];
  if (s < 0) return;                       // padding
  if (s >= num_slots) {
    flag(err, PA_CHECK_SLOT_RANGE);
    return;
  }
  const uint32_t bit = 1u << (uint32_t)(s & 31);
  const uint32_t old = atomicOr(bitmap + (s >> 5), bit);
  if (old & bit) flag(err, PA_CHECK_SLOT_DUPLICATE);
}

// One wavefront per sequence: its length against [0, W * bs], then the table
// entries it uses (j < ceil(n / bs), n clamped as the decode clamps it)
// against the pool.  With query_start_loc (prefill), also the query range.
__global__ __launch_bounds__(kCheckThreads) void check_tables_kernel(const int32_t* __restrict__ tables,
                                                                     const int32_t* __restrict__ ctx,
                                                                     const int32_t* __restrict__ qstart, int32_t B,
                                                                     int32_t W, int32_t bs_log2, int32_t NB,
                                                                     int32_t T, uint32_t* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * (kCheckThreads / 64) + (threadIdx.x >> 6);
  if (b >= B) return;
  const int64_t max_tokens = (int64_t)W << bs_log2;
  const int n = ctx[b];
  if (lane == 0 && (n < 0 || n > max_tokens)) flag(err, PA_CHECK_CONTEXT_RANGE);
  const int nc = n < 0 ? 0 : (n > max_tokens ? (int)max_tokens : n);
  const int nb = (int)(((int64_t)nc + (1 << bs_log2) - 1) >> bs_log2);
  bool bad = false;
  for (int j = lane; j < nb; j += 64) {
    const int32_t e = tables[(size_t)b * W + j];
    bad |= e < 0 || e >= NB;
  }
  if (bad) flag(err, PA_CHECK_TABLE_RANGE);
  if (qstart && lane == 0) {
    const int32_t q0 = qstart[b], q1 = qstart[b + 1];
    bool qbad = q1 < q0 || q0 < 0 || q1 > T || (b == 0 && q0 != 0) || (b == B - 1 && q1 != T);
    qbad |= q1 - q0 > nc;                  // more new queries than tokens: a query at a negative position
    if (qbad) flag(err, PA_CHECK_QUERY_RANGE);
  }
}

int check_desc_basic(const pa_cache_desc* d) {
  if (!d) return PA_ERR_NULL;
  if (d->num_blocks <= 0 || d->num_kv_heads <= 0) return PA_ERR_SHAPE;
  if (d->block_size < 8 || d->block_size > 64 || (d->block_size & (d->block_size - 1))) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int32_t log2_of(int32_t x) {
  int32_t r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

int launch_tables(const int32_t* tables, const int32_t* ctx, const int32_t* qstart, int32_t B, int32_t W,
                  int32_t T, const pa_cache_desc* d, uint32_t* err, hipStream_t s) {
  const uint32_t wpb = kCheckThreads / 64;
  hipLaunchKernelGGL(check_tables_kernel, dim3((uint32_t)((B + wpb - 1) / wpb)), dim3(kCheckThreads), 0, s, tables,
                     ctx, qstart, B, W, log2_of(d->block_size), d->num_blocks, T, err);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

}  // namespace pa

using namespace pa;

extern "C" {

size_t pa_check_write_workspace_bytes(const pa_cache_desc* desc) {
  if (check_desc_basic(desc)) return 0;
  const int64_t slots = (int64_t)desc->num_blocks * desc->block_size;
  return (size_t)((slots + 31) / 32) * sizeof(uint32_t);
}

int pa_check_write(const int64_t* slot_mapping, int32_t num_tokens, const pa_cache_desc* desc, uint32_t* error_word,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc_basic(desc);
  if (st) return st;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (!error_word) return PA_ERR_NULL;
  if (num_tokens == 0) return PA_OK;
  if (!slot_mapping) return PA_ERR_NULL;
  const size_t need = pa_check_write_workspace_bytes(desc);
  if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 3u) != 0) return PA_ERR_ALIGN;
  if (need / sizeof(uint32_t) > 0xffffffffull) return PA_ERR_TOO_LARGE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* bitmap = static_cast<uint32_t*>(workspace);
  const uint32_t words = (uint32_t)(need / sizeof(uint32_t));
  const uint32_t cgrid = (words + kCheckThreads - 1) / kCheckThreads;
  hipLaunchKernelGGL(clear_words_kernel, dim3(cgrid < 1024 ? cgrid : 1024), dim3(kCheckThreads), 0, s, bitmap, words);
  if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  hipLaunchKernelGGL(check_slots_kernel, dim3((uint32_t)((num_tokens + kCheckThreads - 1) / kCheckThreads)),
                     dim3(kCheckThreads), 0, s, slot_mapping, num_tokens,
                     (int64_t)desc->num_blocks * desc->block_size, bitmap, error_word);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int pa_check_decode(const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                    int32_t max_blocks_per_seq, const pa_cache_desc* desc, uint32_t* error_word, void* stream) {
  int st = check_desc_basic(desc);
  if (st) return st;
  if (num_seqs <= 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * desc->block_size > INT32_MAX / 2) return PA_ERR_TOO_LARGE;
  if (!block_tables || !context_lens || !error_word) return PA_ERR_NULL;
  return launch_tables(block_tables, context_lens, nullptr, num_seqs, max_blocks_per_seq, 0, desc, error_word,
                       static_cast<hipStream_t>(stream));
}

int pa_check_prefill(const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start_loc,
                     int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_tokens, const pa_cache_desc* desc,
                     uint32_t* error_word, void* stream) {
  int st = check_desc_basic(desc);
  if (st) return st;
  if (num_seqs <= 0 || max_blocks_per_seq <= 0 || num_tokens < 0) return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * desc->block_size > INT32_MAX / 2) return PA_ERR_TOO_LARGE;
  if (!block_tables || !context_lens || !query_start_loc || !error_word) return PA_ERR_NULL;
  return launch_tables(block_tables, context_lens, query_start_loc, num_seqs, max_blocks_per_seq, num_tokens, desc,
                       error_word, static_cast<hipStream_t>(stream));
}

}  // extern "C"
