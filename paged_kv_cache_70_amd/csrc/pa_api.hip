// C-ABI entry points declared in include/paged_kv.h: argument checks, launch
// planning and kernel launches on the caller's stream.  No allocation, no
// host synchronisation, no state kept between calls, apart from the static
// device scratch area of pa_decode_noalloc (and its per-device address).
#include <limits.h>

#include <atomic>

#include "../../include/paged_kv.h"
#include "pa_internal.h"

namespace pa {

bool dtype_ok(int32_t dtype) { return dtype == PA_F32 || dtype == PA_BF16; }

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return cus[dev];
}
int32_t elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : 2; }

static bool pow2_in(int32_t x, int32_t lo, int32_t hi) {
  return x >= lo && x <= hi && (x & (x - 1)) == 0;
}
static int32_t ilog2(int32_t x) {
  int32_t r = 0;
  while ((1 << r) < x) ++r;
  return r;
}
static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static int check_desc(const pa_cache_desc* d) {
  if (!d) return PA_ERR_NULL;
  if (d->num_blocks <= 0 || d->num_kv_heads <= 0) return PA_ERR_SHAPE;
  if (!dtype_ok(d->dtype)) return PA_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return PA_ERR_UNSUPPORTED;
  if (!pow2_in(d->block_size, 8, 64)) return PA_ERR_UNSUPPORTED;
  if (d->layout != PA_LAYOUT_P09 && d->layout != PA_LAYOUT_VLLM) return PA_ERR_UNSUPPORTED;
  // byte offsets inside the pool are size_t; rows must fit 32-bit lane math
  const int64_t row = (int64_t)d->num_kv_heads * d->head_dim * elem_bytes(d->dtype);
  if (row > INT_MAX) return PA_ERR_TOO_LARGE;
  return PA_OK;
}

// Query heads handled by one wavefront: the largest of 8, 4, 2, 1 dividing G.
static int32_t heads_per_unit(int32_t G) {
  for (int32_t c = 8; c > 1; c >>= 1)
    if (G % c == 0) return c;
  return 1;
}

// Rows of D elements one 16-byte-per-lane load instruction covers.
static int32_t rows_per_wave(const pa_cache_desc* d) {
  const int32_t epv = 16 / elem_bytes(d->dtype);
  return 64 / (d->head_dim / epv);
}

// kv heads per wavefront: as many of a token's (adjacent) kv heads as one
// load instruction covers, so each instruction reads contiguous runs.
static int32_t kv_per_wave(const pa_cache_desc* d) {
  if (d->layout == PA_LAYOUT_VLLM) return 1;   // a token's kv heads are not adjacent there
  int32_t kg = rows_per_wave(d);
  while (d->num_kv_heads % kg) kg >>= 1;
  return kg;
}

// 16-byte loads per K per lane per tile: up to 4, and a tile (tokens per
// load x loads) never crosses a block boundary.
static int32_t tile_unroll(const pa_cache_desc* d) {
  const int32_t tokens_per_load = rows_per_wave(d) / kv_per_wave(d);
  const int32_t u = d->block_size / tokens_per_load;
  return u >= 4 ? 4 : u;
}

// Tokens per split-KV partition chosen without looking at the (device-side)
// context lengths.  Matrix-core path: the largest partition (64 blocks), or
// the whole table when it is shorter.  The persistent kernel streams one unit
// after another without a gap, so long units cost nothing in pipelining, and
// measured on the Llama-3-8B shape (contexts up to 4096 tokens) 1024-token
// partitions beat 256- and 512-token ones by 6-7% in the partial kernel
// alone: fewer partial results are written in the middle of the read stream,
// and the merge has less to read.  Vector-ALU path: 256 tokens, doubled
// while the worst-case number of work units exceeds kTargetUnitsValu.
static constexpr int64_t kTargetUnitsValu = 8192;
// A partition's block-table entries are held one per lane of a wavefront.
static constexpr int32_t kMaxBlocksPerPartition = 64;
static int32_t auto_partition(int32_t B, int32_t W, const pa_cache_desc* d, const DecodePlan& plan) {
  const int64_t max_len = (int64_t)W * d->block_size;
  const int64_t P_max = (int64_t)kMaxBlocksPerPartition * d->block_size;
  if (plan.use_mfma) return (int32_t)(max_len < P_max ? max_len : P_max);
  int64_t P = 256;
  if (P % d->block_size) P = d->block_size;
  {
    const int64_t rows = (int64_t)B * (d->num_kv_heads / kv_per_wave(d)) * plan.nchunks;
    while (P < max_len && P < P_max && rows * ((max_len + P - 1) / P) > kTargetUnitsValu) P *= 2;
  }
  return (int32_t)P;
}

// Wavefronts per workgroup: a unit's tiles are shared by NW wavefronts (merged
// through LDS) when the worst-case unit count alone would leave the chip
// short of wavefronts.
static constexpr int64_t kTargetWaves = 8192;
static int32_t waves_per_unit(int32_t B, const pa_cache_desc* d, const DecodePlan& p) {
  const int64_t units = (int64_t)B * (d->num_kv_heads / p.kv_per_wave) * p.nchunks * p.maxP;
  int32_t nw = 1;
  const int32_t nw_max = p.heads_per_unit <= 4 ? 4 : 2;
  while (nw < nw_max && units * nw < kTargetWaves) nw *= 2;
  return nw;
}

struct Checked {
  DecodePlan plan;
  size_t ws_bytes;
};

static int check_decode_sizes(int32_t B, int32_t H, int32_t W, const pa_cache_desc* d,
                              int32_t partition_size, Checked* out) {
  int st = check_desc(d);
  if (st) return st;
  if (B <= 0 || H <= 0 || W <= 0) return PA_ERR_SHAPE;
  if (H % d->num_kv_heads) return PA_ERR_SHAPE;
  if (partition_size < 0 || (partition_size && partition_size % d->block_size) ||
      partition_size > kMaxBlocksPerPartition * d->block_size)
    return PA_ERR_UNSUPPORTED;
  const int64_t max_len = (int64_t)W * d->block_size;
  if (max_len > INT_MAX / 2) return PA_ERR_TOO_LARGE;
  DecodePlan p;
  const int32_t G = H / d->num_kv_heads;
  p.use_mfma = d->dtype == PA_BF16;
  if (p.use_mfma) {
    // matrix-core kernel: one kv head per unit, its query heads as up to 16
    // product columns
    p.heads_per_unit = G < 16 ? G : 16;
    p.nchunks = (G + 15) / 16;
  } else {
    p.heads_per_unit = heads_per_unit(G);
    p.nchunks = G / p.heads_per_unit;
  }
  p.P = partition_size ? partition_size : auto_partition(B, W, d, p);
  const int64_t maxP = (max_len + p.P - 1) / p.P;
  // grid.y = partitions and grid.z = B are limited to 65535; the merge
  // kernel keeps one fp32 weight per partition in LDS (at most 64 KiB).
  p.kv_per_wave = kv_per_wave(d);
  if ((int64_t)(d->num_kv_heads / p.kv_per_wave) * p.nchunks > INT_MAX || B > 65535 || H > 65535 ||
      maxP > 16384)
    return PA_ERR_TOO_LARGE;
  p.maxP = (int32_t)maxP;
  p.waves_per_unit = p.use_mfma ? 1 : waves_per_unit(B, d, p);
  p.tile_unroll = tile_unroll(d);
  p.vllm = d->layout == PA_LAYOUT_VLLM;
  out->plan = p;
  const int64_t slots = (int64_t)B * H * maxP;
  out->ws_bytes = maxP > 1 ? (size_t)slots * ((size_t)d->head_dim + 2) * sizeof(float) : 0;
  return PA_OK;
}

static int decode_params(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, float scale,
                         int32_t B, int32_t H, int32_t W, const pa_cache_desc* d,
                         void* workspace, size_t workspace_bytes, const Checked& ck,
                         DecodeParams* prm) {
  if (!out || !context_lens) return PA_ERR_NULL;
  if (!aligned16(out)) return PA_ERR_ALIGN;
  if (ck.ws_bytes) {
    if (!workspace || workspace_bytes < ck.ws_bytes) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_ALIGN;
  }
  DecodeParams& p = *prm;
  p.out = out;
  // workspace: [acc: B*H*maxP*D fp32][ml: B*H*maxP*2 fp32]
  const size_t acc_bytes = (size_t)B * H * ck.plan.maxP * d->head_dim * sizeof(float);
  char* ws = static_cast<char*>(workspace);
  p.ws_acc = ck.ws_bytes ? reinterpret_cast<float*>(ws) : nullptr;
  p.ws_ml = ck.ws_bytes ? reinterpret_cast<float*>(ws + acc_bytes) : nullptr;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.tables = block_tables;
  p.ctx = context_lens;
  p.table_rows = nullptr;
  // The kernels take a positive base-2 scale; the sign goes into q.
  const float s2 = scale * 1.4426950408889634f;   // log2(e)
  p.q_mode = s2 > 0.0f ? 0 : (s2 < 0.0f ? 1 : 2);
  p.scale_log2 = s2 > 0.0f ? s2 : (s2 < 0.0f ? -s2 : 1.0f);
  p.B = B;
  p.H = H;
  p.KVH = d->num_kv_heads;
  p.W = W;
  p.NB = d->num_blocks;
  p.bs_log2 = ilog2(d->block_size);
  p.bs_mask = d->block_size - 1;
  p.P = ck.plan.P;
  p.maxP = ck.plan.maxP;
  p.nchunks = ck.plan.nchunks;
  p.max_tokens = W * d->block_size;
  p.SP = 0;
  p.SG = 0;
  p.SPB = 0;
  p.append = 0;
  return PA_OK;
}

// The partial kernel for the cache dtype and layout: bf16 on the matrix cores
// (the P09 or the vLLM-layout tile loads), fp32 on the vector ALUs (either
// layout, chosen by plan.vllm).
static hipError_t launch_partials(const DecodeParams& prm, const pa_cache_desc* desc, const Checked& ck,
                                  hipStream_t s) {
  if (ck.plan.use_mfma)
    return desc->layout == PA_LAYOUT_VLLM ? launch_decode_partials_vllm(prm, desc->head_dim, s)
                                          : launch_decode_partials_mfma(prm, desc->head_dim, s);
  return launch_decode_partials(prm, desc->dtype, desc->head_dim, ck.plan, s);
}

// Shared-prefix folding for a hint of `shared_tokens` leading tokens: whole
// partitions only, and only where a kv head's query heads leave room for at
// least two sequences in the 16 product columns (bf16 matrix-core kernel).
static void set_shared_prefix(DecodeParams& p, int32_t shared_tokens, const Checked& ck) {
  const int32_t G = p.H / p.KVH;
  if (!ck.plan.use_mfma || shared_tokens <= 0 || G >= 16 || 16 % G) return;
  const int32_t tokens = shared_tokens < p.max_tokens ? shared_tokens : p.max_tokens;
  const int32_t SP = tokens / p.P;
  if (SP <= 0) return;
  const int32_t SPB = (SP * p.P + p.bs_mask) >> p.bs_log2;
  // the kernel walks the B x SPB (sequence, entry) pairs it checks with int
  // indices (plus one stride of look-ahead)
  if ((int64_t)p.B * SPB > (1 << 30)) return;
  p.SP = SP;
  p.SG = 16 / G;
  p.SPB = SPB;
}

// Static scratch area of pa_decode_noalloc, for callers that cannot allocate:
// the decode's split-KV partial results.  Each GPU the library runs on holds
// its own copy (at its own address) until the process ends.  In host code
// `scratch` is only a stand-in for that device symbol: its device address is
// looked up per device with hipGetSymbolAddress and used everywhere instead.
static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch area (nullptr on failure).
// The lookup is idempotent, so two threads racing on a device's first call
// both store the same address.
static void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

// Prefill launch shape: query heads per workgroup (the largest of 4, 2, 1
// dividing G) and query tokens per workgroup (4 wavefronts x 32 queries, 16
// for head_dim 256, shared by hg heads).
static int32_t prefill_heads_per_group(int32_t G) {
  return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
}
static int32_t prefill_query_tile(int32_t D, int32_t hg) {
  return (D >= 256 ? 16 : 32) * 4 / hg;
}

}  // namespace pa

using namespace pa;

extern "C" {

int32_t pa_abi_version(void) { return (2 << 16) | 5; }

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer argument";
    case PA_ERR_SHAPE: return "invalid size (non-positive, or num_heads not a multiple of num_kv_heads)";
    case PA_ERR_UNSUPPORTED: return "unsupported head_dim, block_size, dtype or partition size";
    case PA_ERR_WORKSPACE: return "workspace missing or smaller than pa_decode_workspace_bytes()";
    case PA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case PA_ERR_LAUNCH: return "HIP kernel launch failed";
    case PA_ERR_TOO_LARGE: return "sizes exceed the kernels' grid or index limits";
    case PA_ERR_NO_BLOCKS: return "block manager: not enough free blocks";
    case PA_ERR_NO_SEQUENCE: return "block manager: unknown sequence";
    case PA_ERR_NO_MEMORY: return "block manager: host memory ran out (destroy the manager)";
    case PA_ERR_SCRATCH: return "pa_decode_noalloc: more scratch needed than the static area holds, or its address is unavailable";
  }
  return "unknown status";
}

int pa_write_kv(void* k_cache, void* v_cache, const void* k, const void* v,
                const int64_t* slot_mapping, int32_t num_tokens, const pa_cache_desc* desc,
                void* stream) {
  int st = check_desc(desc);
  if (st) return st;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k_cache || !v_cache || !k || !v || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k) || !aligned16(v))
    return PA_ERR_ALIGN;
  const int64_t row_bytes = (int64_t)desc->num_kv_heads * desc->head_dim * elem_bytes(desc->dtype);
  if ((int64_t)num_tokens * (row_bytes / 16) > (int64_t)UINT_MAX - 256) return PA_ERR_TOO_LARGE;
  // the vLLM-layout write spreads a row's 16-byte groups over grid.y, 32 per workgroup
  if (desc->layout == PA_LAYOUT_VLLM && (row_bytes / 16 + 31) / 32 > 65535) return PA_ERR_TOO_LARGE;
  const int64_t num_slots = (int64_t)desc->num_blocks * desc->block_size;
  hipError_t e = desc->layout == PA_LAYOUT_VLLM
                     ? launch_write_kv_vllm(k_cache, v_cache, k, v, slot_mapping, num_tokens, (int32_t)row_bytes,
                                            elem_bytes(desc->dtype), ilog2(desc->block_size), num_slots,
                                            static_cast<hipStream_t>(stream))
                     : launch_write_kv(k_cache, v_cache, k, v, slot_mapping, num_tokens, (int32_t)row_bytes,
                                       num_slots, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                 const pa_cache_desc* desc) {
  Checked ck;
  int st = check_decode_sizes(num_seqs, num_heads, max_blocks_per_seq, desc, 0, &ck);
  return st ? st : ck.plan.P;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                 const pa_cache_desc* desc, int32_t partition_size) {
  Checked ck;
  if (check_decode_sizes(num_seqs, num_heads, max_blocks_per_seq, desc, partition_size, &ck))
    return 0;
  return ck.ws_bytes;
}

size_t pa_decode_append_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                        const pa_cache_desc* desc, int32_t partition_size) {
  Checked ck;
  if (check_decode_sizes(num_seqs, num_heads, max_blocks_per_seq, desc, partition_size, &ck)) return 0;
  // every sequence stores its partials, so one partition per (b, h) at least
  return (size_t)num_seqs * num_heads * ck.plan.maxP * ((size_t)desc->head_dim + 2) * sizeof(float);
}

int pa_decode_append(void* out, const void* q, void* k_cache, void* v_cache, const void* k_new,
                     const void* v_new, const int64_t* slot_mapping, const int32_t* block_tables,
                     const int32_t* cached_lens, float scale, int32_t num_seqs, int32_t num_heads,
                     int32_t max_blocks_per_seq, const pa_cache_desc* desc, int32_t partition_size,
                     void* workspace, size_t workspace_bytes, void* stream) {
  Checked ck;
  int st = check_decode_sizes(num_seqs, num_heads, max_blocks_per_seq, desc, partition_size, &ck);
  if (st) return st;
  if (!q || !k_cache || !v_cache || !k_new || !v_new || !slot_mapping || !block_tables) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return PA_ERR_ALIGN;
  ck.ws_bytes = pa_decode_append_workspace_bytes(num_seqs, num_heads, max_blocks_per_seq, desc, partition_size);
  DecodeParams prm;
  st = decode_params(out, q, k_cache, v_cache, block_tables, cached_lens, scale, num_seqs, num_heads,
                     max_blocks_per_seq, desc, workspace, workspace_bytes, ck, &prm);
  if (st) return st;
  prm.append = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_partials(prm, desc, ck, s) != hipSuccess) return PA_ERR_LAUNCH;
  AppendArgs ap;
  ap.k_new = k_new;
  ap.v_new = v_new;
  ap.slots = slot_mapping;
  ap.k_cache = k_cache;
  ap.v_cache = v_cache;
  ap.num_slots = (int64_t)desc->num_blocks * desc->block_size;
  ap.vllm = desc->layout == PA_LAYOUT_VLLM;
  return launch_decode_merge_append(prm, ap, desc->dtype, desc->head_dim, s) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

static int decode_common(bool partials, bool merge, void* out, const void* q,
                         const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, float scale,
                         int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                         const pa_cache_desc* desc, int32_t partition_size, void* workspace,
                         size_t workspace_bytes, void* stream, int32_t shared_tokens = 0) {
  if (shared_tokens < 0) return PA_ERR_SHAPE;
  Checked ck;
  int st = check_decode_sizes(num_seqs, num_heads, max_blocks_per_seq, desc, partition_size, &ck);
  if (st) return st;
  if (partials) {
    if (!q || !k_cache || !v_cache || !block_tables) return PA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGN;
  }
  DecodeParams prm;
  st = decode_params(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_seqs,
                     num_heads, max_blocks_per_seq, desc, workspace, workspace_bytes, ck, &prm);
  if (st) return st;
  set_shared_prefix(prm, shared_tokens, ck);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (partials) {
    if (launch_partials(prm, desc, ck, s) != hipSuccess) return PA_ERR_LAUNCH;
  }
  if (merge && ck.plan.maxP > 1 &&
      launch_decode_merge(prm, desc->dtype, desc->head_dim, s) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, float scale,
              int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
              const pa_cache_desc* desc, int32_t partition_size, void* workspace,
              size_t workspace_bytes, void* stream) {
  return decode_common(true, true, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                       num_seqs, num_heads, max_blocks_per_seq, desc, partition_size, workspace,
                       workspace_bytes, stream);
}

int pa_decode_partials(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens, float scale,
                       int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                       const pa_cache_desc* desc, int32_t partition_size, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return decode_common(true, false, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                       num_seqs, num_heads, max_blocks_per_seq, desc, partition_size, workspace,
                       workspace_bytes, stream);
}

int pa_decode_shared_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, float scale,
                            int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                            int32_t shared_tokens, const pa_cache_desc* desc, int32_t partition_size,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(true, true, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                       num_seqs, num_heads, max_blocks_per_seq, desc, partition_size, workspace,
                       workspace_bytes, stream, shared_tokens);
}

int pa_decode_partials_shared_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* context_lens, float scale,
                                     int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                     int32_t shared_tokens, const pa_cache_desc* desc, int32_t partition_size,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(true, false, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                       num_seqs, num_heads, max_blocks_per_seq, desc, partition_size, workspace,
                       workspace_bytes, stream, shared_tokens);
}

int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                      const pa_cache_desc* desc, int32_t partition_size, void* stream) {
  Checked ck;
  int st = check_decode_sizes(num_seqs, num_heads, max_blocks_per_seq, desc, partition_size, &ck);
  if (st) return st;
  if (ck.ws_bytes > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGN;
  void* ws = nullptr;
  if (ck.ws_bytes) {
    ws = scratch_address();
    if (!ws) return PA_ERR_SCRATCH;
  }
  return decode_common(true, true, out, q, k_cache, v_cache, block_tables, context_lens, scale, num_seqs,
                       num_heads, max_blocks_per_seq, desc, partition_size, ws, ck.ws_bytes, stream);
}

int pa_decode_merge(void* out, const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                    int32_t max_blocks_per_seq, const pa_cache_desc* desc,
                    int32_t partition_size, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return decode_common(false, true, out, nullptr, nullptr, nullptr, nullptr, context_lens, 1.0f,
                       num_seqs, num_heads, max_blocks_per_seq, desc, partition_size, workspace,
                       workspace_bytes, stream);
}

// Prefill launch geometry shared by the workspace query and the call.
//   bf16: the matrix-core kernel; workspace = its work plan.
//   fp32: one vector-ALU decode per query row over the first (position + 1)
//   tokens of its sequence; workspace = per-row contexts and table rows, then
//   the decode's partial results (partitions of 64 blocks).
struct PrefillShape {
  int32_t hg, nchunks, tq;
  int64_t max_tiles;
  size_t ws_bytes;
  size_t meta_bytes;      // fp32: the per-row arrays ahead of the decode workspace
  Checked dec;            // fp32: the decode plan over num_tokens rows
};

static int prefill_shape(int32_t B, int32_t H, int32_t W, int32_t T, const pa_cache_desc* d, PrefillShape* out) {
  int st = check_desc(d);
  if (st) return st;
  if (B <= 0 || H <= 0 || W <= 0 || T < 0) return PA_ERR_SHAPE;
  if (H % d->num_kv_heads) return PA_ERR_SHAPE;
  PrefillShape p{};
  if (d->dtype == PA_F32) {
    if (T > 65535) return PA_ERR_TOO_LARGE;
    const int64_t max_len = (int64_t)W * d->block_size;
    const int32_t P = (int32_t)(max_len < 64LL * d->block_size ? max_len : 64LL * d->block_size);
    st = check_decode_sizes(T > 0 ? T : 1, H, W, d, P, &p.dec);
    if (st) return st;
    p.meta_bytes = ((size_t)T * 2 * sizeof(int32_t) + 15) & ~(size_t)15;
    p.ws_bytes = p.meta_bytes + p.dec.ws_bytes;
    if (p.ws_bytes == 0) p.ws_bytes = 16;
    *out = p;
    return PA_OK;
  }
  const int32_t G = H / d->num_kv_heads;
  p.hg = prefill_heads_per_group(G);
  p.nchunks = G / p.hg;
  p.tq = prefill_query_tile(d->head_dim, p.hg);
  // (sequence, query tile) pairs: sum_b ceil(L_b / tq) <= ceil(T / tq) + B;
  // a plan entry packs the sequence and the tile into 16 bits each
  p.max_tiles = ((int64_t)T + p.tq - 1) / p.tq + B;
  if (B > 65536 || ((int64_t)T + p.tq - 1) / p.tq > 65536 ||
      p.max_tiles * d->num_kv_heads * p.nchunks > INT_MAX)
    return PA_ERR_TOO_LARGE;
  p.ws_bytes = kPrefillHeaderBytes + (size_t)p.max_tiles * sizeof(uint32_t);
  *out = p;
  return PA_OK;
}

size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                  int32_t num_tokens, const pa_cache_desc* desc) {
  PrefillShape p;
  return prefill_shape(num_seqs, num_heads, max_blocks_per_seq, num_tokens, desc, &p) ? 0 : p.ws_bytes;
}

int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens,
               const int32_t* query_start_loc, float scale, int32_t num_seqs, int32_t num_heads,
               int32_t max_blocks_per_seq, int32_t num_tokens, const pa_cache_desc* desc,
               void* workspace, size_t workspace_bytes, void* stream) {
  const int32_t B = num_seqs, H = num_heads, W = max_blocks_per_seq;
  PrefillShape shp;
  int st = prefill_shape(B, H, W, num_tokens, desc, &shp);
  if (st) return st;
  const int64_t max_len = (int64_t)W * desc->block_size;
  if (max_len > INT_MAX / 2) return PA_ERR_TOO_LARGE;
  if (num_tokens == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
    return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGN;
  if (!workspace || workspace_bytes < shp.ws_bytes) return PA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return PA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (desc->dtype == PA_F32) {
    int32_t* rows_ctx = static_cast<int32_t*>(workspace);
    int32_t* rows_tbl = rows_ctx + num_tokens;
    char* dec_ws = static_cast<char*>(workspace) + shp.meta_bytes;
    DecodeParams prm;
    st = decode_params(out, q, k_cache, v_cache, block_tables, rows_ctx, scale, num_tokens, H, W, desc,
                       dec_ws, workspace_bytes - shp.meta_bytes, shp.dec, &prm);
    if (st) return st;
    prm.table_rows = rows_tbl;
    if (launch_prefill_rows(query_start_loc, context_lens, B, num_tokens, (int32_t)max_len, rows_ctx, rows_tbl, s) !=
        hipSuccess)
      return PA_ERR_LAUNCH;
    if (launch_decode_partials(prm, desc->dtype, desc->head_dim, shp.dec.plan, s) != hipSuccess) return PA_ERR_LAUNCH;
    if (shp.dec.plan.maxP > 1 && launch_decode_merge(prm, desc->dtype, desc->head_dim, s) != hipSuccess)
      return PA_ERR_LAUNCH;
    return PA_OK;
  }
  PrefillParams p;
  p.hg = shp.hg;
  p.nchunks = shp.nchunks;
  p.tq = shp.tq;
  p.max_tiles = (int32_t)shp.max_tiles;
  p.tickets = static_cast<int32_t*>(workspace);
  p.plan = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + kPrefillHeaderBytes);
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.tables = block_tables;
  p.ctx = context_lens;
  p.qstart = query_start_loc;
  const float s2 = scale * 1.4426950408889634f;   // log2(e)
  p.q_mode = s2 > 0.0f ? 0 : (s2 < 0.0f ? 1 : 2);
  p.scale_log2 = s2 > 0.0f ? s2 : (s2 < 0.0f ? -s2 : 1.0f);
  p.B = B;
  p.H = H;
  p.KVH = desc->num_kv_heads;
  p.W = W;
  p.NB = desc->num_blocks;
  p.T = num_tokens;
  p.bs_log2 = ilog2(desc->block_size);
  p.bs_mask = desc->block_size - 1;
  p.max_tokens = (int32_t)max_len;
  p.vllm = desc->layout == PA_LAYOUT_VLLM ? 1 : 0;
  return launch_prefill_mfma(p, desc->head_dim, s) == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"
