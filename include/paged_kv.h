/*
 * paged_kv.h — C ABI of the paged KV-cache write, paged decode attention and
 * paged (varlen, causal) prefill attention for AMD Instinct MI355X (gfx950).
 *
 * The operations are the ones defined on the page "P09 · Paged KV 写入 +
 * decode attention（参考实现）" (kuanzhou.online), sections 题面速览 and
 * 框架视角 · shape trace, and described as a kernel on "PagedAttention
 * kernel：paged KV cache 与 block table" (inference-learning-path.pages.dev),
 * sections 直接答案 and 深入原理 (v1/v2 partitioning):
 *
 *   cache layout   [num_blocks, block_size, num_kv_heads, head_dim]
 *   write          cache[slot / bs][slot % bs] = k[i]   (slot < 0: padding, skipped)
 *   decode         per sequence b with n = context_lens[b]:
 *                  K_b = cache[block_tables[b, :ceil(n/bs)]] flattened to tokens, first n rows
 *                  out[b,h] = softmax(scale * q[b,h] . K_b[:, h / (H/KVH)]) . V_b[:, h / (H/KVH)]
 *                  scores, softmax and the weighted sum in fp32; out in q's dtype.
 *
 * Conventions for every entry point
 *   - Pointers marked "device" are HIP device pointers (any allocation the
 *     current device can access); "host" pointers are ordinary host memory.
 *   - Every tensor is dense row-major (C-contiguous) with the stated shape and
 *     at least 16-byte aligned.  The caller owns every buffer; the library
 *     allocates nothing and keeps no state between calls (the one exception
 *     is pa_decode_noalloc's static device scratch area).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *     the legacy default stream).  No call synchronises the host.
 *   - Return value: PA_OK (0) or a negative pa_status.  Argument errors are
 *     detected on the host before anything is enqueued; PA_ERR_LAUNCH reports
 *     a failed kernel launch.  pa_status_string() names each code.
 *   - Device-side preconditions (not checked on the host, since that would
 *     need a device-to-host copy; the opt-in pa_check_* calls test them on
 *     the device): non-negative slots are < num_blocks *
 *     block_size and pairwise distinct; for j < ceil(n_b / bs),
 *     0 <= block_tables[b, j] < num_blocks; 0 <= context_lens[b] <=
 *     max_blocks_per_seq * block_size.  The kernels stay memory-safe when they
 *     are violated: a slot outside the cache is skipped like padding, a table
 *     entry outside the pool contributes no tokens, and a context length is
 *     clamped to [0, max_blocks_per_seq * block_size].  Duplicate slots leave
 *     one of the written rows (unspecified which).
 */
#ifndef PAGED_KV_H
#define PAGED_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v, the caches and out (all share one). */
typedef enum pa_dtype {
  PA_F32 = 0,  /* IEEE binary32 */
  PA_BF16 = 1  /* bfloat16 (upper half of binary32); out is rounded to nearest even */
} pa_dtype;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,         /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,        /* a size is negative/zero where it must be positive, or H % KVH != 0 */
  PA_ERR_UNSUPPORTED = -3,  /* head_dim not in {64,128,256}, block_size not in {8,16,32,64}, unknown dtype
                               or layout, a layout/dtype pair an entry point does not implement,
                               or a partition size that is not a positive multiple of block_size
                               or spans more than 64 blocks */
  PA_ERR_WORKSPACE = -4,    /* workspace NULL or smaller than pa_decode_workspace_bytes() */
  PA_ERR_ALIGN = -5,        /* a tensor pointer is not 16-byte aligned */
  PA_ERR_LAUNCH = -6,       /* the HIP runtime rejected a kernel launch */
  PA_ERR_TOO_LARGE = -7,    /* sizes overflow the kernels' 32-bit grid/index limits */
  PA_ERR_NO_BLOCKS = -8,    /* block manager: not enough free blocks (nothing was changed) */
  PA_ERR_NO_SEQUENCE = -9,  /* block manager: unknown sequence id */
  PA_ERR_NO_MEMORY = -10,   /* block manager: host memory ran out inside a call that changes the
                               manager; its state is then unspecified: destroy it */
  PA_ERR_SCRATCH = -11      /* pa_decode_noalloc: the call needs more than the library's static
                               scratch area of PA_NOALLOC_SCRATCH_BYTES, or the device address of
                               that area could not be obtained */
} pa_status;

/* Memory layout of the two caches. */
typedef enum pa_layout {
  /* "P09 · Paged KV 写入 + decode attention", 题面速览: both caches
     [num_blocks, block_size, num_kv_heads, head_dim]. */
  PA_LAYOUT_P09 = 0,
  /* vLLM's, "PagedAttention kernel：paged KV cache 与 block table", 深入原理:
     k_cache [num_blocks, num_kv_heads, head_dim / x, block_size, x] with x
     elements = 16 bytes (8 for bf16, 4 for fp32), v_cache [num_blocks,
     num_kv_heads, head_dim, block_size].  Supported by pa_write_kv, the
     decode entry points and pa_prefill, in both dtypes. */
  PA_LAYOUT_VLLM = 1
} pa_layout;

/* Geometry of the paged cache (k_cache and v_cache share it). */
typedef struct pa_cache_desc {
  int32_t num_blocks;    /* NB: physical blocks in the pool, > 0 */
  int32_t block_size;    /* bs: tokens per block, one of 8, 16, 32, 64 */
  int32_t num_kv_heads;  /* KVH, > 0 */
  int32_t head_dim;      /* D, one of 64, 128, 256 */
  int32_t dtype;         /* a pa_dtype */
  int32_t layout;        /* a pa_layout */
} pa_cache_desc;

/*
 * pa_write_kv — scatter new tokens' K/V rows into the paged cache, in place.
 * "P09 · Paged KV 写入 + decode attention" (kuanzhou.online), 题面速览 (写) and
 * shape trace write_kv steps 1-4: for every i with slot_mapping[i] >= 0,
 * k_cache[slot / bs, slot % bs, :, :] = k[i] and the same for v.  Negative
 * slots are padding (CUDA-graph padded batches use -1) and write nothing.
 * The copy is bit-exact.
 *
 *   k_cache, v_cache  device, in desc->layout ([NB, bs, KVH, D] for PA_LAYOUT_P09)
 *                     of desc->dtype, updated in place
 *   k, v              device, [num_tokens, KVH, D] of desc->dtype
 *   slot_mapping      device, [num_tokens] int64 flat slot = block * bs + offset
 *   num_tokens        T >= 0; T == 0 enqueues nothing and returns PA_OK
 *   desc              host, cache geometry
 *   stream            hipStream_t
 * Returns PA_OK once the kernel is enqueued (asynchronous: nothing waits for
 * it), or PA_ERR_NULL / PA_ERR_SHAPE / PA_ERR_UNSUPPORTED / PA_ERR_ALIGN,
 * PA_ERR_TOO_LARGE when T * KVH * D * elem / 16 exceeds 32 bits (or, in
 * PA_LAYOUT_VLLM, a row holds more than 65535 * 32 sixteen-byte groups), and
 * PA_ERR_LAUNCH.  Slots at or past num_blocks * bs are skipped like padding;
 * valid slots must be distinct: two tokens with the same slot leave an
 * unspecified mix of their rows.
 */
int pa_write_kv(void* k_cache, void* v_cache, const void* k, const void* v,
                const int64_t* slot_mapping, int32_t num_tokens,
                const pa_cache_desc* desc, void* stream);

/*
 * pa_decode_partition_size — the split-KV partition length (tokens) that
 * pa_decode uses when it is passed partition_size == 0.  Partitioning is the
 * "v2" scheme of "PagedAttention kernel：paged KV cache 与 block table",
 * 深入原理: a long context is cut into partitions processed in parallel and
 * merged afterwards.  Depends only on its arguments (no device access).
 * Returns a positive multiple of desc->block_size, or a negative pa_status.
 */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_heads,
                                 int32_t max_blocks_per_seq, const pa_cache_desc* desc);

/*
 * pa_decode_workspace_bytes — size of the fp32 workspace pa_decode needs for
 * the per-partition partial results (max, sum, accumulator per query head) of
 * the split-KV path; 0 when no sequence can span two partitions.
 * partition_size 0 selects pa_decode_partition_size().  Returns 0 for invalid
 * arguments.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads,
                                 int32_t max_blocks_per_seq, const pa_cache_desc* desc,
                                 int32_t partition_size);

/*
 * pa_decode — paged decode attention, one query per sequence.
 * "P09 · Paged KV 写入 + decode attention" (kuanzhou.online), 题面速览
 * (decode 读) and shape trace decode steps 1-7; online softmax over the block
 * table as on "PagedAttention kernel：paged KV cache 与 block table", 直接答案.
 * Enqueues the partial kernel and, when some sequence spans more than one
 * partition, the merge kernel (the same as pa_decode_partials followed by
 * pa_decode_merge).
 *
 *   out                 device, [B, H, D] of desc->dtype (written)
 *   q                   device, [B, H, D] of desc->dtype
 *   k_cache, v_cache    device, in desc->layout ([NB, bs, KVH, D] for PA_LAYOUT_P09)
 *                       of desc->dtype
 *   block_tables        device, [B, max_blocks_per_seq] int32; only the first
 *                       ceil(context_lens[b] / bs) entries of row b are read
 *   context_lens        device, [B] int32, tokens of each sequence (0 gives zeros)
 *   scale               multiplies q.k before the softmax (typically 1/sqrt(D))
 *   num_seqs, num_heads B > 0, H > 0 with H % KVH == 0
 *   max_blocks_per_seq  table width W > 0
 *   desc                host, cache geometry
 *   partition_size      tokens per split-KV partition: 0 = automatic, else a
 *                       positive multiple of block_size, at most 64 * block_size
 *   workspace           device, >= pa_decode_workspace_bytes(...) bytes, no
 *                       initial contents required; may be NULL only when the
 *                       requirement is 0.  Calls that share a workspace must
 *                       not run concurrently.
 *   stream              hipStream_t
 *
 * bf16 caches run on the matrix cores (16-token tiles, up to 16 query heads of
 * a kv head per product); fp32 caches on the vector ALUs.
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, float scale,
              int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
              const pa_cache_desc* desc, int32_t partition_size,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_partials — first half of a two-pass decode (same arguments as
 * pa_decode): every (sequence, kv head, partition) folds its tokens with an
 * online softmax.  Sequences that fit in one partition (and n == 0) get their
 * final output written to `out`; the others leave fp32 partial results in
 * `workspace` for pa_decode_merge (or for a merge of partitions computed
 * elsewhere).  Workspace layout, with P the partition size in use and
 * maxP = ceil(max_blocks_per_seq * bs / P):
 *   acc  fp32 [B, H, maxP, D] at byte 0,
 *   ml   fp32 [B, H, maxP, 2] right after acc: (m, l) per partition,
 * where partition p of sequence b and head h holds acc = sum_t 2^(s_t - m) v_t
 * and l = sum_t 2^(s_t - m) over its tokens t, s_t = scale * log2(e) * q.k_t
 * and m a reference at least the largest s_t minus 8 (not necessarily the
 * maximum), so that acc / l is the softmax-weighted V of the partition alone.
 */
int pa_decode_partials(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens, float scale,
                       int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                       const pa_cache_desc* desc, int32_t partition_size,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_shared_prefix — pa_decode for a batch whose tables may begin with
 * the same blocks: sequences that share a prompt prefix point their tables at
 * the same physical blocks for it ("PagedAttention kernel：paged KV cache 与
 * block table", 面试官追问 on prefix sharing).  Same arguments and result as
 * pa_decode, plus
 *   shared_tokens   >= 0: a hint that table rows may equal row 0 over their
 *                   first shared_tokens / block_size entries.  The leading
 *                   floor(min(shared_tokens, W * bs) / P) whole partitions
 *                   (P: the partition size in use) are folded for up to
 *                   16 / G sequences at once (G = num_heads / num_kv_heads
 *                   query heads of one kv head side by side as the 16 matrix
 *                   columns), so each shared block is read once per group
 *                   instead of once per sequence.
 * The device checks every row: a sequence takes part only if its first
 * entries over those partitions equal row 0's and its context extends past
 * them; every other sequence, and any call where G does not divide 16 or is
 * 16 or more, the fp32 dtype, or more than 4096 sequences, is decoded as by
 * pa_decode.  The result therefore never depends on the hint being right: a
 * wrong hint costs only the check.  Output equals pa_decode's within fp32
 * rounding (per-column softmax state; the lazy rescale may fire at other
 * tiles).  Workspace: pa_decode_workspace_bytes.  Errors as pa_decode, plus
 * PA_ERR_SHAPE for shared_tokens < 0.
 */
int pa_decode_shared_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, float scale,
                            int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                            int32_t shared_tokens, const pa_cache_desc* desc, int32_t partition_size,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_partials_shared_prefix — the first half of pa_decode_shared_prefix
 * (as pa_decode_partials is of pa_decode); pa_decode_merge finishes it.
 */
int pa_decode_partials_shared_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* context_lens, float scale,
                                     int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                     int32_t shared_tokens, const pa_cache_desc* desc, int32_t partition_size,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_merge — second half of pa_decode: for every sequence spanning
 * more than one partition, combines the partial results of pa_decode_partials
 * (max-rescaled sums: out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p)
 * and writes `out`.  Must follow pa_decode_partials on the same stream with
 * the same arguments.
 */
int pa_decode_merge(void* out, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                    const pa_cache_desc* desc, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_prefill_workspace_bytes — size of the device workspace pa_prefill needs.
 * bf16: its work plan, 48 bytes (ticket counters) plus 4 per (sequence,
 * query tile) pair (bounded by num_tokens / tile + num_seqs).  fp32: 8 bytes per query row
 * plus the split-KV partial results of one decode per query row (as
 * pa_decode_workspace_bytes for num_tokens sequences, partitions of 64
 * blocks).  Depends only on its arguments; 0 for invalid arguments.
 */
size_t pa_prefill_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                  int32_t num_tokens, const pa_cache_desc* desc);

/*
 * pa_prefill — paged attention of a packed (varlen) batch of new query tokens,
 * causal within each sequence (prefill, or one chunk of a chunked prefill).
 * "P09 · Paged KV 写入 + decode attention" (kuanzhou.online) asks for this
 * varlen prefill in 面试官追问 & 对照源码 without defining it; this is the
 * reading its 细节 supports (decode needs no causal mask only because its one
 * query is the newest token):
 *   sequence b owns q rows query_start_loc[b] .. query_start_loc[b+1] - 1
 *   (L_b of them); they are its last L_b tokens, whose K/V rows are already in
 *   the cache (pa_write_kv first), so query i is token p = n_b - L_b + i with
 *   n_b = context_lens[b]; it attends to tokens 0 .. p of the sequence,
 *   gathered through block_tables exactly as pa_decode does:
 *   out[row, h] = softmax_{j <= p}(scale * q[row, h] . K_b[j, kvh]) . V_b[:, kvh],
 *   kvh = h / (H / KVH); fp32 scores and softmax, out rounded to bf16.
 * With L_b = 1 for every b this is pa_decode.
 *
 *   out               device, [num_tokens, H, D] in the cache dtype (written;
 *                     rows of no sequence are left untouched)
 *   q                 device, [num_tokens, H, D] in the cache dtype
 *   k_cache, v_cache  device, [NB, bs, KVH, D] (PA_LAYOUT_P09), or for bf16
 *                     in PA_LAYOUT_VLLM K [NB, KVH, D/8, bs, 8] and
 *                     V [NB, KVH, D, bs]
 *   block_tables      device, [B, max_blocks_per_seq] int32; row b's first
 *                     ceil(n_b / bs) entries are read
 *   context_lens      device, [B] int32, n_b (new tokens included)
 *   query_start_loc   device, [B + 1] int32, non-decreasing from 0 to num_tokens
 *   scale             multiplies q.k before the softmax
 *   num_tokens        T >= 0 (T == 0 enqueues nothing)
 *   desc              host, cache geometry.  bf16 runs the matrix-core
 *                     kernel, in either layout; fp32 runs one vector-ALU
 *                     decode per query row over its first (position + 1)
 *                     tokens (a plain path for small fp32 workloads:
 *                     num_tokens <= 65535), PA_LAYOUT_P09 only
 *                     (PA_ERR_UNSUPPORTED otherwise)
 *   workspace         device, >= pa_prefill_workspace_bytes(...) bytes, no
 *                     initial contents required.  Calls that share a
 *                     workspace must not run concurrently.
 * bf16 enqueues a one-workgroup planning kernel (the work list, heaviest
 * first) and the attention kernel, whose workgroups draw work from that list;
 * fp32 enqueues a per-row kernel (each row's context and table row), the
 * decode partial kernel and, if needed, the merge.
 * Device-side preconditions as for pa_decode, plus L_b <= n_b (queries at
 * negative positions, if any, get zeros) and query_start_loc as stated
 * (entries are clamped to [0, num_tokens]).  Memory safety holds when they
 * are violated, but unlike pa_decode a table entry outside the pool is not
 * masked out: its rows read as zeros and take part in the softmax.
 */
int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens,
               const int32_t* query_start_loc, float scale, int32_t num_seqs, int32_t num_heads,
               int32_t max_blocks_per_seq, int32_t num_tokens, const pa_cache_desc* desc,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Host block manager with prefix sharing (CPU only; no device access).  It
 * hands out the physical blocks whose ids fill block_tables, slot_mapping and
 * context_lens for the calls above.  Sources: the third page's BlockManager
 * (a pool of fixed-size blocks, each keeping its token ids and a hash of them
 * chained with its prefix's hash, a hash -> block map, a queue of free ids,
 * allocate reporting the cached prefix) and "PagedAttention kernel：paged KV
 * cache 与 block table", 面试官追问 (sequences sharing a prompt prefix point
 * at the same blocks for it).  Semantics where the pages stop:
 *   - a full block is shared under the chained key h_i = FNV-1a-64 over the
 *     8-byte little-endian words (h_{i-1}, t_0 .. t_{bs-1}), h_{-1} = all ones,
 *     when the stored tokens are equal too; partial blocks are private; a
 *     block is registered for sharing once it is full;
 *   - a new sequence reuses cached blocks from its start up to the first
 *     one that is not cached; every later block is new;
 *   - blocks are reference-counted; at count 0 a block joins the back of the
 *     free queue keeping its key (a later sequence can revive it); new blocks
 *     come from the front (initially 0 .. NB-1), evicting a cached block there;
 *   - an operation that cannot get its blocks returns PA_ERR_NO_BLOCKS and
 *     changes nothing.
 * Slot of position p of a sequence: table[p / bs] * bs + p % bs.
 * Not thread-safe: use one manager per thread or lock around calls.
 */
typedef struct pa_block_manager pa_block_manager;

/* A manager of num_blocks blocks of block_size tokens; NULL for non-positive
 * sizes or if memory runs out.  Free it with pa_bm_destroy.  No call lets a
 * C++ exception out: a failed host allocation returns PA_ERR_NO_MEMORY. */
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager* bm);

/* New sequence holding tokens[0 .. n).  *seq_id receives its id (0, 1, 2, ...
 * in creation order); *cached_tokens (may be NULL) the number of leading
 * tokens whose blocks were already cached (a multiple of block_size). */
int pa_bm_add_sequence(pa_block_manager* bm, const int64_t* tokens, int32_t n, int64_t* seq_id,
                       int32_t* cached_tokens);

/* Appends one token; *slot receives its slot (for pa_write_kv). */
int pa_bm_append(pa_block_manager* bm, int64_t seq_id, int64_t token, int64_t* slot);

/* One decode step: appends tokens[i] to sequence seq_ids[i] for every i (each
 * id at most once) and writes the slots -- the step's slot_mapping -- into
 * slots[i].  All or nothing: an unknown id (PA_ERR_NO_SEQUENCE), a repeated
 * id (PA_ERR_SHAPE) or too few free blocks (PA_ERR_NO_BLOCKS) changes
 * nothing. */
int pa_bm_append_batch(pa_block_manager* bm, const int64_t* seq_ids, const int64_t* tokens, int32_t n,
                       int64_t* slots);

/* Releases a sequence's blocks (shared blocks stay with their other users). */
int pa_bm_free_sequence(pa_block_manager* bm, int64_t seq_id);

/* Tokens of a sequence, or a negative pa_status. */
int32_t pa_bm_length(const pa_block_manager* bm, int64_t seq_id);

/* Blocks in the free queue (cached ones included), or a negative pa_status. */
int32_t pa_bm_num_free(const pa_block_manager* bm);

/* The sequence's block table into out[0 .. capacity); *num_blocks receives
 * its length (PA_ERR_SHAPE, with *num_blocks set, if capacity is short). */
int pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out, int32_t capacity,
                      int32_t* num_blocks);

/* Slots of positions start .. start + count - 1 of a sequence into out. */
int pa_bm_slots(const pa_block_manager* bm, int64_t seq_id, int32_t start, int32_t count, int64_t* out);

/* Host arrays for a batch: block_tables [num_seqs, max_blocks_per_seq]
 * (rows padded with `fill`) and context_lens [num_seqs], the inputs of
 * pa_decode / pa_prefill once copied to the device. */
int pa_bm_fill_tables(const pa_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                      int32_t max_blocks_per_seq, int32_t fill, int32_t* block_tables,
                      int32_t* context_lens);

/*
 * pa_decode_append — one decode step that appends each sequence's new token:
 * the same result as pa_write_kv of the new rows followed by pa_decode, in two
 * kernels instead of three.  The write and gather steps of "P09 · Paged KV 写入
 * + decode attention" (题面速览, decode shape trace) and the partition merge of
 * "PagedAttention kernel：paged KV cache 与 block table" (深入原理, v2).
 *
 * Sequence b owns one new token (its K/V rows k_new[b], v_new[b]) unless
 * slot_mapping[b] < 0 or >= num_blocks * bs.  It attends to its cached_lens[b]
 * cached tokens, gathered through block_tables as in pa_decode, plus the new
 * token. The output equals pa_decode with context_lens[b] = cached_lens[b] + 1
 * after the new token was written at slot_mapping[b], which must be the slot
 * of position cached_lens[b] in b's table.  The partial kernel reads only the
 * cached tokens; the merge kernel reads the new token from k_new / v_new, folds
 * it into the softmax and copies its rows, bit for bit, into the slot.
 *
 *   out, q            device, [num_seqs, H, D] of desc->dtype
 *   k_cache, v_cache  device, desc->layout; the new rows are written into them
 *   k_new, v_new      device, [num_seqs, KVH, D] of desc->dtype
 *   slot_mapping      device, [num_seqs] int64
 *   cached_lens       device, [num_seqs] int32, tokens already in the cache
 *                     (clamped to [0, max_blocks_per_seq * bs])
 *   workspace         device, >= pa_decode_append_workspace_bytes(...) bytes
 *   others            as for pa_decode
 * Returns as pa_decode (PA_ERR_WORKSPACE when the workspace is missing or
 * short).  Valid slots must be distinct.  Calls sharing a workspace must not
 * run concurrently.
 */
size_t pa_decode_append_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                                        const pa_cache_desc* desc, int32_t partition_size);
int pa_decode_append(void* out, const void* q, void* k_cache, void* v_cache, const void* k_new,
                     const void* v_new, const int64_t* slot_mapping, const int32_t* block_tables,
                     const int32_t* cached_lens, float scale, int32_t num_seqs, int32_t num_heads,
                     int32_t max_blocks_per_seq, const pa_cache_desc* desc, int32_t partition_size,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc — pa_decode for callers that cannot allocate device
 * memory (code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments without the
 * workspace, and the same result, bit for bit, as pa_decode with the same
 * partition size.  The split-KV partial results go to a static device array
 * of PA_NOALLOC_SCRATCH_BYTES held by the library on every GPU it runs on
 * until the process ends; the call itself allocates nothing and calls no
 * allocating runtime or library routine.
 *   - The need is pa_decode_workspace_bytes(...) for the same sizes; a call
 *     that needs more returns PA_ERR_SCRATCH before anything is enqueued.
 *   - The area's device address is looked up once per device, on that
 *     device's first call (the stream's device must be current, as for
 *     every entry point); a failed lookup returns PA_ERR_SCRATCH.
 *   - Every call on one GPU shares that GPU's area and leaves its partial
 *     results there; none need be cleared (a call writes every slot it
 *     reads).  Calls that overlap on one GPU (concurrent streams, or
 *     threads) race: order them on one stream.
 * Other errors as pa_decode.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int32_t num_seqs, int32_t num_heads, int32_t max_blocks_per_seq,
                      const pa_cache_desc* desc, int32_t partition_size, void* stream);

/*
 * Checked mode (opt-in).  The device-side preconditions above are not tested
 * by the write, decode and prefill kernels, which stay memory-safe when they
 * are broken and report nothing -- the silent failures "P09 · Paged KV 写入 +
 * decode attention" warns of: a -1 slot used as an index overwrites the last
 * row with no error or warning (直觉与类比), and garbage table entries give an
 * index error or silently wrong K/V (易错点).  The pa_check_* calls enqueue
 * kernels that test them and OR one bit per kind of violation into
 * *error_word (device, uint32, set with atomics; the caller zeroes it before
 * the checks it wants to collect and reads it after they ran).  Enqueue them
 * on the same stream before (or instead of) the call they guard; they read
 * only what that call reads and write only *error_word and their workspace.
 */
typedef enum pa_check_flag {
  PA_CHECK_SLOT_RANGE = 1,       /* a slot >= num_blocks * block_size (negative slots are padding) */
  PA_CHECK_SLOT_DUPLICATE = 2,   /* two tokens with the same valid slot */
  PA_CHECK_TABLE_RANGE = 4,      /* block_tables[b, j] outside [0, num_blocks) for some j < ceil(n_b / bs) */
  PA_CHECK_CONTEXT_RANGE = 8,    /* context_lens[b] < 0 or > max_blocks_per_seq * block_size */
  PA_CHECK_QUERY_RANGE = 16      /* prefill: query_start_loc not non-decreasing from 0 to num_tokens, or a
                                    sequence with more new queries than tokens (L_b > n_b) */
} pa_check_flag;

/* Bytes of the slot bitmap pa_check_write needs: one bit per cache slot
 * (num_blocks * block_size), rounded up to 4-byte words; 0 for an invalid desc. */
size_t pa_check_write_workspace_bytes(const pa_cache_desc* desc);

/* Checks a write's slot_mapping [num_tokens] (device int64): sets
 * PA_CHECK_SLOT_RANGE and PA_CHECK_SLOT_DUPLICATE.  workspace: device,
 * 4-byte aligned, >= pa_check_write_workspace_bytes(desc), no initial contents
 * (a fill kernel clears it).  Calls sharing a workspace must not overlap.
 * Returns PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE,
 * PA_ERR_ALIGN, PA_ERR_TOO_LARGE or PA_ERR_LAUNCH; num_tokens == 0 enqueues nothing. */
int pa_check_write(const int64_t* slot_mapping, int32_t num_tokens, const pa_cache_desc* desc,
                   uint32_t* error_word, void* workspace, size_t workspace_bytes, void* stream);

/* Checks a decode's block_tables [B, W] and context_lens [B] (device int32;
 * for pa_decode_append pass its cached_lens): sets PA_CHECK_CONTEXT_RANGE and
 * PA_CHECK_TABLE_RANGE, reading only the entries the decode reads. */
int pa_check_decode(const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                    int32_t max_blocks_per_seq, const pa_cache_desc* desc, uint32_t* error_word, void* stream);

/* pa_check_decode plus the prefill's query_start_loc [B + 1] (device int32)
 * against num_tokens and the context lengths: also sets PA_CHECK_QUERY_RANGE. */
int pa_check_prefill(const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start_loc,
                     int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_tokens, const pa_cache_desc* desc,
                     uint32_t* error_word, void* stream);

/*
 * pa_measure_read — a measurement helper, not a step of the method: reads
 * the `bytes` bytes of `buf` once with 16-byte loads (non-temporal when
 * `nontemporal` is nonzero, as the decode's KV loads are): workgroups_per_cu
 * workgroups of 256 threads per compute unit, each streaming one contiguous
 * chunk of the buffer.  Its rate, timed beside the decode, is the
 * streaming-read ceiling of the same byte count on the same device.
 *   buf    device, 16-byte aligned, bytes a multiple of 16 (0: nothing enqueued)
 *   sink   device, one uint32 the kernel may write (it keeps the loads live)
 * Returns PA_OK, PA_ERR_NULL, PA_ERR_ALIGN, PA_ERR_SHAPE (bytes not a multiple
 * of 16, workgroups_per_cu outside 1..64), PA_ERR_TOO_LARGE (a chunk of 2 GiB
 * or more) or PA_ERR_LAUNCH.
 */
int pa_measure_read(const void* buf, size_t bytes, int32_t workgroups_per_cu, int32_t nontemporal,
                    uint32_t* sink, void* stream);

/*
 * pa_measure_mfma — a measurement helper, not a step of the method: every
 * wavefront of workgroups_per_cu workgroups of 256 threads per compute unit
 * runs `iters` rounds of 4 independent v_mfma_f32_32x32x16_bf16 products on
 * register operands (32,768 flops each; no memory traffic).  Its rate, timed
 * beside the prefill, is the matrix-core ceiling the device sustains.
 *   sink   device, one uint32 the kernel may write (it keeps the products live)
 * Returns PA_OK, PA_ERR_NULL, PA_ERR_SHAPE (iters <= 0, workgroups_per_cu
 * outside 1..8) or PA_ERR_LAUNCH.
 */
int pa_measure_mfma(int32_t iters, int32_t workgroups_per_cu, uint32_t* sink, void* stream);

/* Static, NUL-terminated name of a pa_status code ("unknown status" otherwise). */
const char* pa_status_string(int status);

/* ABI version of this header: (major << 16) | minor (2.0: pa_cache_desc.layout;
 * 2.1: fp32 prefill, pa_prefill_workspace_bytes takes max_blocks_per_seq;
 * 2.2: pa_decode_shared_prefix, pa_decode_partials_shared_prefix;
 * 2.3: pa_decode_append, pa_decode_append_workspace_bytes;
 * 2.4: pa_decode_noalloc, PA_ERR_SCRATCH; 2.5: checked mode (pa_check_*),
 * pa_measure_read). */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_H */
