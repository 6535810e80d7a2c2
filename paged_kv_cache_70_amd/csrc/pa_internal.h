// Internal interface between the C-ABI entry points (pa_api.hip) and the
// kernel launchers (pa_write.hip, pa_decode.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Everything the decode kernels need, passed by value as the kernel argument.
struct DecodeParams {
  void* out;               // [B, H, D] of the element type
  float* ws_acc;           // [B, H, maxP, D] fp32 partial accumulators
  float* ws_ml;            // [B, H, maxP, 2]  fp32 partial (max, sum), max in log2 units
  const void* q;           // [B, H, D]
  const void* k_cache;     // [NB, bs, KVH, D]
  const void* v_cache;
  const int32_t* tables;   // [B, W]
  const int32_t* ctx;      // [B]
  const int32_t* table_rows;  // nullptr: sequence b reads table row b; else row table_rows[b] (fp32 kernel)
  float scale_log2;        // |scale| * log2(e) > 0: scores are kept in base-2 exponent units
  int32_t q_mode;          // 0: q as given, 1: negate q (scale < 0), 2: zero q (scale == 0)
  int32_t B, H, KVH, W, NB;
  int32_t bs_log2, bs_mask;
  int32_t P;               // tokens per partition, multiple of bs
  int32_t maxP;            // partitions reserved per (b, h) in the workspace
  int32_t nchunks;         // head chunks per kv head (G / heads-per-unit)
  int32_t max_tokens;      // W * bs: context lengths are clamped to this
  // Shared prefix (bf16 persistent kernel only; 0 elsewhere): the first SP
  // partitions of every sequence whose first SPB table entries equal row 0's
  // and whose context extends past them are folded SG sequences per unit
  // (their G heads side by side as the product's 16 columns).
  int32_t SP, SG, SPB;
  // Append step: every unit stores its (acc, m, l) partial, a sequence's only
  // partition included, for the merge that folds in the new token.
  int32_t append;
};

// The append step's new token per sequence (row b of k_new / v_new is
// sequence b's), written into the caches by the merge that folds it in.
struct AppendArgs {
  const void* k_new;         // [B, KVH, D]
  const void* v_new;
  const int64_t* slots;      // [B]; negative or >= num_slots: no new token
  void* k_cache;             // the caches, in the layout below
  void* v_cache;
  int64_t num_slots;         // NB * bs
  int32_t vllm;              // 0: [NB, bs, KVH, D]; 1: vLLM's K and V blocks
};

// Launch-shape choices made on the host (pure functions of the sizes).
struct DecodePlan {
  int32_t use_mfma;        // bf16: matrix-core kernel (16-token tiles, up to 16 heads per unit)
  int32_t heads_per_unit;  // query heads sharing one K/V stream in one wavefront
  int32_t nchunks;         // G / heads_per_unit
  int32_t P;               // partition length in tokens
  int32_t maxP;            // ceil(W * bs / P)
  int32_t kv_per_wave;     // kv heads whose rows one load instruction covers (KG)
  int32_t waves_per_unit;  // wavefronts of a workgroup sharing one unit's tiles (NW)
  int32_t tile_unroll;     // 16-byte loads per K (and per V) per tile and lane
  int32_t vllm;            // caches in vLLM's layout (vector-ALU kernel: fp32 only)
};

// Prefill workspace header: one ticket counter per class of workgroups (the
// dies), then the number of plan entries; the plan follows at 48 bytes.
constexpr int kTicketClasses = 8;
constexpr size_t kPrefillHeaderBytes = 48;
static_assert((kTicketClasses + 1) * 4 <= kPrefillHeaderBytes, "prefill header");

// Paged prefill (bf16, matrix cores): a packed batch of new queries per
// sequence, causal over the sequence's paged K/V.
struct PrefillParams {
  void* out;               // [T, H, D] bf16
  const void* q;           // [T, H, D] bf16
  const void* k_cache;     // [NB, bs, KVH, D] bf16
  const void* v_cache;
  const int32_t* tables;   // [B, W]
  const int32_t* ctx;      // [B] tokens of each sequence, its new ones included
  const int32_t* qstart;   // [B + 1] first q row of each sequence
  float scale_log2;        // |scale| * log2(e) > 0
  int32_t q_mode;          // 0: q as given, 1: negate q (scale < 0), 2: zero q (scale == 0)
  int32_t B, H, KVH, W, NB, T;
  int32_t bs_log2, bs_mask;
  int32_t max_tokens;      // W * bs: context lengths are clamped to this
  int32_t hg;              // query heads per workgroup (4, 2 or 1, dividing G)
  int32_t nchunks;         // G / hg
  int32_t tq;              // query tokens per workgroup (128 / hg)
  int32_t max_tiles;       // bound on the (sequence, query tile) pairs: T / tq + B
  uint32_t* plan;          // workspace: [max_tiles] (sequence << 16 | query tile), heaviest first
  int32_t* tickets;        // workspace: [c] next unit of class c < kTicketClasses, [kTicketClasses] plan entries
  int32_t vllm;            // caches in vLLM's layout (K [NB, KVH, D/8, bs, 8], V [NB, KVH, D, bs])
};

bool dtype_ok(int32_t dtype);
int device_cus();        // compute units of the current device (0 if the runtime cannot tell)
int32_t elem_bytes(int32_t dtype);

hipError_t launch_write_kv(void* k_cache, void* v_cache, const void* k, const void* v,
                           const int64_t* slots, int32_t T, int32_t row_bytes,
                           int64_t num_slots, hipStream_t stream);

hipError_t launch_decode_partials(const DecodeParams& prm, int32_t dtype, int32_t D,
                                  const DecodePlan& plan, hipStream_t stream);

hipError_t launch_decode_partials_mfma(const DecodeParams& prm, int32_t D, hipStream_t stream);

// Caches in vLLM's layout (K [NB, KVH, D/x, bs, x], V [NB, KVH, D, bs]).
hipError_t launch_write_kv_vllm(void* k_cache, void* v_cache, const void* k, const void* v,
                                const int64_t* slots, int32_t T, int32_t row_bytes, int32_t elem_bytes,
                                int32_t bs_log2, int64_t num_slots, hipStream_t stream);
hipError_t launch_decode_partials_vllm(const DecodeParams& prm, int32_t D, hipStream_t stream);

hipError_t launch_prefill_mfma(const PrefillParams& prm, int32_t D, hipStream_t stream);

// fp32 prefill as one decode per query: per query row, its context (position
// + 1, 0 at a negative position) and its sequence's table row.
hipError_t launch_prefill_rows(const int32_t* qstart, const int32_t* ctx, int32_t B, int32_t T,
                               int32_t max_tokens, int32_t* ctx_out, int32_t* rows_out, hipStream_t stream);

hipError_t launch_decode_merge(const DecodeParams& prm, int32_t dtype, int32_t D,
                               hipStream_t stream);
hipError_t launch_decode_merge_append(const DecodeParams& prm, const AppendArgs& ap, int32_t dtype, int32_t D,
                                      hipStream_t stream);

}  // namespace pa
