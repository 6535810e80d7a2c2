// Paged decode attention for gfx950: split-KV partial kernel + partition merge.
//
// Operation: "P09 · Paged KV 写入 + decode attention" (kuanzhou.online),
// 题面速览 (decode 读) and the decode shape trace: sequence b reads the first
// n = context_lens[b] rows through block_tables[b, :ceil(n / bs)], query head h
// uses kv head h / (H / KVH), and out = softmax(scale * q . K^T) . V in fp32.
// The block-by-block online softmax is the scheme of "PagedAttention kernel：
// paged KV cache 与 block table" (直接答案, 代码); splitting long contexts into
// partitions merged afterwards is its "v2" (深入原理).
//
// Work decomposition (one 64-lane wavefront per work unit):
//   unit = (partition p, kv head, chunk of GC query heads of that kv head, sequence b)
//   The wavefront streams the partition's tokens tile by tile.  A tile is TT
//   consecutive tokens inside one physical block; every lane issues U 16-byte
//   loads for K and U for V per tile.  LPT = D / (elements per 16 B) lanes
//   hold one token's D-row (256 contiguous bytes for D = 128 bf16), so one
//   load instruction fetches RPW = 64 / LPT whole token rows.
//   Each K row is loaded once and used by all GC query heads (the GQA group
//   shares its kv head).  Partial dot products are summed across the LPT
//   lanes of a row with DPP row rotations / quad permutes (no LDS traffic).
//   Every row of lanes keeps its own running (max, sum, accumulator) for its
//   tokens; the RPW row states are combined once at the end of the unit.
//   Scores are kept in base-2 units (q.k * scale * log2 e) so that every
//   exponential is one v_exp_f32.
// A sequence that fits in one partition writes `out` directly; longer ones
// write fp32 partials that the merge kernel combines:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
//
// Masking uses selects (never multiply-by-zero), so rows beyond n in the last
// block, whatever they hold (NaN included), cannot reach the output.
#include <math.h>

#include <type_traits>

#include "pa_internal.h"

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// element types: 16-byte vectors of fp32 (4 values) or bf16 (8 values)
// ---------------------------------------------------------------------------
struct F32 {
  static constexpr int EPV = 4;
  static constexpr uint32_t kSignMask = 0x80000000u;   // sign bit of each 32-bit word
  // partial dot product of this lane's 4 q values with 4 k values
  __device__ static __forceinline__ float dot(const u32x4& q, const u32x4& k) {
    float s = __uint_as_float(q[0]) * __uint_as_float(k[0]);
    s = fmaf(__uint_as_float(q[1]), __uint_as_float(k[1]), s);
    s = fmaf(__uint_as_float(q[2]), __uint_as_float(k[2]), s);
    s = fmaf(__uint_as_float(q[3]), __uint_as_float(k[3]), s);
    return s;
  }
  __device__ static __forceinline__ void widen(const u32x4& v, float (&f)[EPV]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
  __device__ static __forceinline__ void store(void* out, size_t idx, const float (&f)[EPV]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(f[i]);
    *reinterpret_cast<u32x4*>(static_cast<float*>(out) + idx) = w;
  }
};

struct BF16 {
  static constexpr int EPV = 8;
  static constexpr uint32_t kSignMask = 0x80008000u;   // sign bits of both bf16 halves
  // bf16 x bf16 products are exact in fp32; v_dot2 adds two of them per step.
  __device__ static __forceinline__ float dot(const u32x4& q, const u32x4& k) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // Copy the lanes to scalars before the bit cast: a bit cast applied to
      // an ext-vector element directly is lowered to element 0 by this clang.
      const uint32_t qa = q[i], ka = k[i];
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qa),
                                          __builtin_bit_cast(bf16x2, ka), s, false);
    }
    return s;
  }
  // a bf16 is the high half of an fp32: widening is a shift / mask
  __device__ static __forceinline__ void widen(const u32x4& v, float (&f)[EPV]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  // round to nearest even (IEEE conversion semantics of __bf16)
  __device__ static __forceinline__ void store(void* out, size_t idx, const float (&f)[EPV]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x2 pr;
      pr[0] = (__bf16)f[2 * i];
      pr[1] = (__bf16)f[2 * i + 1];
      w[i] = __builtin_bit_cast(uint32_t, pr);
    }
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + idx) = w;
  }
};

// ---------------------------------------------------------------------------
// cross-lane helpers
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over the LPT consecutive lanes that hold one token row; every lane of the
// row receives the total.  Within 16 lanes: row_ror 8 and 4 (or the half-row
// mirror for 8 lanes) fold the row onto quads, two quad permutes finish it.
template <int LPT>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(LPT == 4 || LPT == 8 || LPT == 16 || LPT == 32 || LPT == 64, "row width");
  if constexpr (LPT >= 16) {
    x += dpp<0x128>(x);  // row_ror:8
    x += dpp<0x124>(x);  // row_ror:4
  } else if constexpr (LPT == 8) {
    x += dpp<0x141>(x);  // row_half_mirror
  }
  x += dpp<0x4E>(x);     // quad_perm [2,3,0,1]
  x += dpp<0xB1>(x);     // quad_perm [1,0,3,2]
  if constexpr (LPT >= 32) x += __shfl_xor(x, 16);
  if constexpr (LPT >= 64) x += __shfl_xor(x, 32);
  return x;
}

// row_sum for N independent values, one reduction step across all of them at
// a time, so consecutive DPP operations never depend on each other.
template <int LPT, int N>
__device__ __forceinline__ void row_sum_all(float* x) {
  static_assert(LPT == 4 || LPT == 8 || LPT == 16 || LPT == 32 || LPT == 64, "row width");
  if constexpr (LPT >= 16) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp<0x128>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp<0x124>(x[i]);
  } else if constexpr (LPT == 8) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += dpp<0x141>(x[i]);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp<0x4E>(x[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] += dpp<0xB1>(x[i]);
  if constexpr (LPT >= 32) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __shfl_xor(x[i], 16);
  }
  if constexpr (LPT >= 64) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] += __shfl_xor(x[i], 32);
  }
}

// Combine over the RPW rows of the wavefront (lanes LPT apart).
template <int LPT>
__device__ __forceinline__ float rows_max(float x) {
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
template <int LPT>
__device__ __forceinline__ float rows_sum(float x) {
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Word 3 of a buffer resource for gfx9-family targets (raw, untyped loads).
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// ---------------------------------------------------------------------------
// K2: split-KV partial kernel
// ---------------------------------------------------------------------------
// The running softmax state of a row is kept against a reference maximum m
// (base-2 units) that is raised only when a score exceeds it by more than
// kRescaleSlack: every term 2^(s - m) stays below 2^kRescaleSlack, the
// accumulators hold sum 2^(s - m) v and sum 2^(s - m), and the final ratio is
// the same softmax.  Raising m rescales the accumulators by 2^(m_old - m_new).
constexpr float kRescaleSlack = 8.0f;

// VL: the caches are in vLLM's layout ("PagedAttention kernel：paged KV cache 与
// block table", 深入原理): K [NB, KVH, D/x, bs, x] with x = 16 bytes of
// elements, so the lane's 16-byte piece c of a token's K row is group c of the
// (block, kv head)'s [D/x][bs][x] region; V [NB, KVH, D, bs], so its EPV
// elements of a token are EPV 4-byte-or-smaller reads bs elements apart (fp32:
// four 4-byte loads per piece).  The tile, the lanes' rows and the fold are
// the same as in the P09 layout; only the load offsets change (KG = 1: a
// token's kv heads are not adjacent there).
template <typename E, int D, int GC, int U, int KG, int NW, bool VL = false>
__global__ __launch_bounds__(64 * NW) void decode_partial_kernel(const DecodeParams prm) {
  constexpr int EPV = E::EPV;
  constexpr int LPT = D / EPV;       // lanes per (token, kv head) row of D elements
  constexpr int RPW = 64 / LPT;      // rows per load instruction
  static_assert(KG >= 1 && RPW % KG == 0, "kv heads per wavefront");
  constexpr int TR = RPW / KG;       // tokens per load instruction
  constexpr int TT = TR * U;         // tokens per tile
  constexpr int ESZ = 16 / EPV;      // bytes per element
  constexpr int NSTATE = GC * (EPV + 2);

  // Grid: x = (kv-head group, head chunk) fastest, so the groups covering one
  // block's token rows are dispatched together; y = partition; z = sequence.
  // The NW wavefronts of a workgroup share the unit and take its tiles in turn.
  const int p = blockIdx.y;
  const int b = blockIdx.z;
  const int kvg = blockIdx.x / prm.nchunks;
  const int chunk = blockIdx.x - kvg * prm.nchunks;

  int n = prm.ctx[b];
  n = n < 0 ? 0 : (n > prm.max_tokens ? prm.max_tokens : n);
  const int nparts = (n + prm.P - 1) / prm.P;
  if (p >= (nparts > 0 ? nparts : 1)) return;           // uniform over the workgroup
  const int t_begin = p * prm.P;
  const int t_end = min(n, t_begin + prm.P);

  const int wave = NW > 1 ? (int)(threadIdx.x >> 6) : 0;
  const int lane = threadIdx.x & 63;
  const int r = lane / LPT;          // row of this lane within a load
  const int c = lane - r * LPT;      // 16-byte piece of the D-row
  // Row r covers kv head kvg * KG + r % KG of token r / KG: the KG heads of
  // one token are adjacent in memory, so a load instruction reads TR runs of
  // KG * D contiguous elements.
  const int kvh = kvg * KG + r % KG;
  const int tr = r / KG;
  const int G = prm.H / prm.KVH;
  const int h0 = kvh * G + chunk * GC;

  // This lane's slice of the GC queries.  The host passes a positive scale:
  // for a negative one the queries are negated here, for zero they are zeroed.
  u32x4 qv[GC];
  {
    const char* qb = static_cast<const char*>(prm.q) +
                     ((size_t)(b * prm.H + h0) * D + (size_t)c * EPV) * ESZ;
    const uint32_t flip = prm.q_mode == 1 ? E::kSignMask : 0u;
    const uint32_t keep = prm.q_mode == 2 ? 0u : 0xffffffffu;
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      qv[g] = load16(qb + (size_t)g * D * ESZ);
#pragma unroll
      for (int i = 0; i < 4; ++i) qv[g][i] = (qv[g][i] ^ flip) & keep;
    }
  }
  const float cs = prm.scale_log2;   // > 0

  float m[GC], mneg[GC], l[GC], acc[GC][EPV];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    m[g] = -INFINITY;
    mneg[g] = 0.0f;                  // -m, or 0 while m is -inf
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[g][e] = 0.0f;
  }

  const uint32_t row_bytes = (uint32_t)prm.KVH * D * ESZ;         // token stride in a block
  const size_t blk_bytes = (size_t)row_bytes << prm.bs_log2;
  const uint32_t tile_bytes = row_bytes * TT;
  // Per-lane byte offset inside a tile: fixed for the whole unit, so the loads
  // need no per-tile vector address arithmetic.
  const uint32_t lane_off = (uint32_t)kvh * D * ESZ + (uint32_t)c * 16 + (uint32_t)tr * row_bytes;
  const char* kc = static_cast<const char*>(prm.k_cache);
  const char* vc = static_cast<const char*>(prm.v_cache);
  const int32_t* tbl = prm.tables + (size_t)(prm.table_rows ? prm.table_rows[b] : b) * prm.W;

  // Block-table entries of this partition, one per lane (a partition spans at
  // most 64 blocks): each tile takes its physical block id with v_readlane, so
  // the tile loop issues no scalar loads and no conditional vector loads.
  // Only entries below ceil(n / bs) are read.
  const int j_first = t_begin >> prm.bs_log2;
  const int j_end = (t_end + prm.bs_mask) >> prm.bs_log2;       // one past the last entry used
  const int tbl_v = (j_first + lane < j_end) ? tbl[j_first + lane] : 0;

  // Tile state: U K-vectors and U V-vectors per lane, double buffered so that
  // the next tile's loads are in flight while this tile is folded.  A tile is
  // read through a buffer resource based at its first row (built in scalar
  // registers); a block outside the pool gets an empty resource, whose loads
  // return zeros without touching memory.
  u32x4 kA[U], vA[U], kB[U], vB[U];

  // vLLM layout: per-lane offsets inside a (block, kv head) region, and the
  // region's byte size (the same for K and V: D * bs elements)
  const uint32_t vl_region = (uint32_t)D * ESZ << prm.bs_log2;
  const uint32_t vl_k_off = (((uint32_t)c << prm.bs_log2) + (uint32_t)tr) * 16;
  const uint32_t vl_v_off = (((uint32_t)(c * EPV) << prm.bs_log2) + (uint32_t)tr) * ESZ;
  auto load_tile = [&](int tile, u32x4 (&kr)[U], u32x4 (&vr)[U]) -> bool {
    const int phys = __builtin_amdgcn_readlane(tbl_v, (tile >> prm.bs_log2) - j_first);
    const bool ok = (unsigned)phys < (unsigned)prm.NB;
    if constexpr (VL) {
      static_assert(KG == 1 && E::EPV == 4, "vLLM layout: fp32, one kv head per row of lanes");
      // one resource over the (block, kv head) region, empty outside the pool
      // (KG = 1: kvh is the same for every lane)
      const size_t boff = (size_t)(ok ? phys : 0) * blk_bytes + (size_t)kvh * vl_region;
      const int nrec = ok ? (int)vl_region : 0;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + boff), (short)0, nrec, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + boff), (short)0, nrec, kRsrcWord3);
      const uint32_t t0 = (uint32_t)(tile & prm.bs_mask);     // the tile's first row in its block
#pragma unroll
      for (int u = 0; u < U; ++u)
        kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, vl_k_off, (t0 + u * TR) * 16, 0);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vr[u][e] = __builtin_amdgcn_raw_buffer_load_b32(rv, vl_v_off + ((uint32_t)e << prm.bs_log2) * ESZ,
                                                          (t0 + u * TR) * ESZ, 0);
      __builtin_amdgcn_sched_barrier(0);
      return ok;
    }
    const size_t off = (size_t)(ok ? phys : 0) * blk_bytes + (size_t)(tile & prm.bs_mask) * row_bytes;
    const int nrec = ok ? (int)tile_bytes : 0;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + off), (short)0, nrec, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + off), (short)0, nrec, kRsrcWord3);
#pragma unroll
    for (int u = 0; u < U; ++u) kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off, u * TR * row_bytes, 0);
#pragma unroll
    for (int u = 0; u < U; ++u) vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off, u * TR * row_bytes, 0);
    // Keep the scheduler from hoisting the previous tile's arithmetic (which
    // must wait for its own loads) above these loads.
    __builtin_amdgcn_sched_barrier(0);
    return ok;
  };

  // Fold one tile into the running state.  A full tile has every row valid
  // (unless its block is outside the pool: then ok is false and its scores
  // are -inf, its V rows zero).  The MASKED variant handles the tile holding
  // the sequence end: rows past nvalid get a -inf score and a zero V row, by
  // selection.
  auto fold_tile = [&](auto masked, bool ok, int nvalid, const u32x4 (&kr)[U], const u32x4 (&vr)[U]) {
    constexpr bool MASKED = decltype(masked)::value;
    float s[U][GC];                  // q.k, then scaled to base-2 units
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < GC; ++g) s[u][g] = E::dot(qv[g], kr[u]);
    row_sum_all<LPT, U * GC>(&s[0][0]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = ok && (!MASKED || (u * TR + tr) < nvalid);
#pragma unroll
      for (int g = 0; g < GC; ++g) s[u][g] = valid ? s[u][g] * cs : -INFINITY;
    }
    // Raise the reference maxima only when some score outgrows them.  The
    // maxima are taken over the same scaled scores the exponentials use, so a
    // lone score gives exactly 2^0 = 1.
    float mt[GC];
    bool raise = false;
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      float x = s[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) x = fmaxf(x, s[u][g]);
      mt[g] = x;
      raise |= mt[g] > m[g] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(raise)) {             // wavefront-uniform
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        if (mt[g] > m[g]) {
          const float corr = exp2_fast(m[g] - mt[g]);        // 0 while m is -inf
          m[g] = mt[g];
          mneg[g] = -mt[g];
          l[g] *= corr;
#pragma unroll
          for (int e = 0; e < EPV; ++e) acc[g][e] *= corr;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[EPV];
      E::widen(vr[u], vf);
      if constexpr (MASKED) {
        const bool valid = (u * TR + tr) < nvalid;
#pragma unroll
        for (int e = 0; e < EPV; ++e) vf[e] = valid ? vf[e] : 0.0f;
      }
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        const float pr = exp2_fast(s[u][g] + mneg[g]);
        l[g] += pr;
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[g][e] = fmaf(pr, vf[e], acc[g][e]);
      }
    }
  };

  // This wavefront's tiles are w, w + NW, w + 2 NW, ... of the unit: full
  // tiles in a loop of pairs (A/B buffers swap roles every half, with a single
  // loop exit so that each buffer keeps its registers), then the odd full tile
  // and the unit's one partial tile (sequence end), if it is this wave's.
  const int ntok = t_end - t_begin;
  const int nfull = ntok > 0 ? ntok / TT : 0;
  const int rem = ntok > 0 ? ntok - nfull * TT : 0;
  const int ntiles = nfull + (rem ? 1 : 0);
  const int my_full = nfull > wave ? (nfull - wave + NW - 1) / NW : 0;
  const int my_tiles = ntiles > wave ? (ntiles - wave + NW - 1) / NW : 0;
  const bool my_rem = my_tiles > my_full;
  if (my_tiles > 0) {
    // j-th tile of this wave; past its last one the last one is fetched again
    // (cache hit) so that every step issues its loads.
    auto tile_at = [&](int j) { return t_begin + (wave + min(j, my_tiles - 1) * NW) * TT; };
    bool okA = load_tile(tile_at(0), kA, vA), okB;
    const int npairs = my_full >> 1;
    for (int ip = 0; ip < npairs; ++ip) {
      okB = load_tile(tile_at(2 * ip + 1), kB, vB);
      fold_tile(std::false_type{}, okA, TT, kA, vA);
      okA = load_tile(tile_at(2 * ip + 2), kA, vA);
      fold_tile(std::false_type{}, okB, TT, kB, vB);
    }
    if (my_full & 1) {
      okB = load_tile(tile_at(my_full), kB, vB);
      fold_tile(std::false_type{}, okA, TT, kA, vA);
      if (my_rem) fold_tile(std::true_type{}, okB, rem, kB, vB);
    } else if (my_rem) {
      fold_tile(std::true_type{}, okA, rem, kA, vA);
    }
  }

  // Combine the TR row states of each kv head (rows LPT * KG lanes apart),
  // then, with several wavefronts, the wavefronts' states through LDS.
  float M[GC], L[GC];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    M[g] = rows_max<LPT * KG>(m[g]);
    const float f = (m[g] == -INFINITY) ? 0.0f : exp2_fast(m[g] - M[g]);
    L[g] = rows_sum<LPT * KG>(l[g] * f);
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[g][e] = rows_sum<LPT * KG>(acc[g][e] * f);
  }
  if constexpr (NW > 1) {
    extern __shared__ float lds_state[];             // [NW][64 lanes][NSTATE]
    float* mine = lds_state + ((size_t)wave * 64 + lane) * NSTATE;
    if (wave > 0 && tr == 0) {
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        mine[g * (EPV + 2)] = M[g];
        mine[g * (EPV + 2) + 1] = L[g];
#pragma unroll
        for (int e = 0; e < EPV; ++e) mine[g * (EPV + 2) + 2 + e] = acc[g][e];
      }
    }
    __syncthreads();
    if (wave > 0) return;
    if (tr == 0) {
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        float Mx = M[g];
#pragma unroll
        for (int w = 1; w < NW; ++w) Mx = fmaxf(Mx, lds_state[((size_t)w * 64 + lane) * NSTATE + g * (EPV + 2)]);
        const float f0 = (M[g] == -INFINITY) ? 0.0f : exp2_fast(M[g] - Mx);
        L[g] *= f0;
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[g][e] *= f0;
#pragma unroll
        for (int w = 1; w < NW; ++w) {
          const float* o = lds_state + ((size_t)w * 64 + lane) * NSTATE + g * (EPV + 2);
          const float fw = (o[0] == -INFINITY) ? 0.0f : exp2_fast(o[0] - Mx);
          L[g] = fmaf(o[1], fw, L[g]);
#pragma unroll
          for (int e = 0; e < EPV; ++e) acc[g][e] = fmaf(o[2 + e], fw, acc[g][e]);
        }
        M[g] = Mx;
      }
    }
  }

  const bool single = nparts <= 1 && !prm.append;
  if (tr == 0) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      const size_t bh = (size_t)b * prm.H + h0 + g;
      if (single) {
        const float inv = L[g] > 0.0f ? 1.0f / L[g] : 0.0f;
        float o[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) o[e] = acc[g][e] * inv;
        E::store(prm.out, bh * D + (size_t)c * EPV, o);
      } else {
        const size_t slot = bh * prm.maxP + p;
        float* dst = prm.ws_acc + slot * D + (size_t)c * EPV;
#pragma unroll
        for (int e = 0; e < EPV; e += 4)
          *reinterpret_cast<float4*>(dst + e) = make_float4(acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]);
        if (c == 0) *reinterpret_cast<float2*>(prm.ws_ml + slot * 2) = make_float2(M[g], L[g]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// K3: partition merge
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

// Partition rows of one (sequence, head) that the merge-append kernel loads
// before the context length arrives: the first min(maxP, kMergeEarlyRows).
// They lie inside the workspace's maxP >= 1 rows of that (sequence, head)
// whatever the length; rows past the sequence's partitions hold stale or
// unwritten values and are dropped by selects (never multiplied by a zero
// weight, which would keep a stale NaN).  The plain merge kernel does not
// load early: a quarter of its wavefronts (single-partition sequences) leave
// at once, and early loads there measured slower.
constexpr int kMergeEarlyRows = 8;

typedef float mf4 __attribute__((ext_vector_type(4)));

template <int D, int PPI, int KPRE>
__device__ __forceinline__ void early_rows(const float* acc, const float* ml, int early, int sub, int dl, int lane,
                                           mf4 (&pre)[KPRE], float2& mlpre) {
  // Every lane loads (at a row index clamped to early - 1 < maxP) and then
  // selects: loads under a lane condition each get a branch of their own,
  // and the compiler waits for them inside it.
#pragma unroll
  for (int k = 0; k < KPRE; ++k) {
    const int i = sub + PPI * k;
    const mf4 v = *reinterpret_cast<const mf4*>(acc + (size_t)min(i, early - 1) * D + dl);
    pre[k] = i < early ? v : mf4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const float2 m = *reinterpret_cast<const float2*>(ml + (size_t)min(lane, early - 1) * 2);
  mlpre = lane < early ? m : make_float2(-INFINITY, 0.0f);
}

// The rows of the round starting at partition r0 (cnt of them): in round 0
// the early rows come from pre / mlpre, the rest are loaded now.  Rows i <
// PPI * KPRE of round 0 are early rows or lie past maxP >= cnt.
template <int D, int PPI, int KMAX, int KPRE>
__device__ __forceinline__ void round_rows(const float* acc, const float* ml, int r0, int cnt, int early, int sub,
                                           int dl, int lane, const mf4 (&pre)[KPRE], float2 mlpre, mf4 (&a)[KMAX],
                                           float2& mlv) {
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int i = sub + PPI * k;
    if (k < KPRE && r0 == 0)
      a[k] = i < cnt ? pre[k] : mf4{0.0f, 0.0f, 0.0f, 0.0f};
    else
      a[k] = i < cnt ? *reinterpret_cast<const mf4*>(acc + (size_t)(r0 + i) * D + dl) : mf4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  if (r0 == 0 && lane < early)
    mlv = lane < cnt ? mlpre : make_float2(-INFINITY, 0.0f);
  else
    mlv = lane < cnt ? *reinterpret_cast<const float2*>(ml + (size_t)(r0 + lane) * 2) : make_float2(-INFINITY, 0.0f);
}

template <typename E, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const DecodeParams prm) {
  // One wavefront per (sequence, head).  A partial accumulator row is D fp32
  // = D / 4 lanes x 16 B, so one load instruction brings PPI = 256 / D rows;
  // lane (sub, dl) accumulates rows sub, sub + PPI, ... at d = dl .. dl + 3.
  // The (max, sum) pairs are read one per lane, R partitions per round; the
  // accumulator loads of a round are issued before its maxima are reduced.
  constexpr int LPP = D / 4;
  constexpr int PPI = 64 / LPP;
  constexpr int KMAX = PPI * 16 <= 64 ? 16 : 64 / PPI;   // loads per lane per round
  constexpr int R = PPI * KMAX;                          // partitions per round (<= 64)
  typedef float f4 __attribute__((ext_vector_type(4)));
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  int n = prm.ctx[b];
  n = n < 0 ? 0 : (n > prm.max_tokens ? prm.max_tokens : n);
  const int nparts = (n + prm.P - 1) / prm.P;
  if (nparts <= 1) return;                 // written by the partial kernel
  const int lane = threadIdx.x;
  const int sub = lane / LPP;
  const int dl = (lane % LPP) * 4;
  const size_t bh = (size_t)b * prm.H + h;
  const float* ml = prm.ws_ml + bh * prm.maxP * 2;
  const float* acc = prm.ws_acc + bh * prm.maxP * D;

  float Mrun = -INFINITY, Lrun = 0.0f;     // running (max, sum) over rounds, wave-uniform
  f4 o = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int r0 = 0; r0 < nparts; r0 += R) {
    const int cnt = min(R, nparts - r0);
    f4 a[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const int i = sub + PPI * k;
      a[k] = i < cnt ? *reinterpret_cast<const f4*>(acc + (size_t)(r0 + i) * D + dl) : f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const float2 mlv = lane < cnt ? *reinterpret_cast<const float2*>(ml + (size_t)(r0 + lane) * 2)
                                  : make_float2(-INFINITY, 0.0f);
    const float M = fmaxf(Mrun, wave_max(mlv.x));
    const float w = mlv.x == -INFINITY ? 0.0f : exp2_fast(mlv.x - M);
    const float fo = Mrun == -INFINITY ? 0.0f : exp2_fast(Mrun - M);
    Lrun = Lrun * fo + wave_sum(w * mlv.y);
    o *= fo;
    Mrun = M;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) o += __shfl(w, sub + PPI * k) * a[k];
  }
  // rows sub = 0 .. PPI-1 hold disjoint partition sets of the same d range
#pragma unroll
  for (int off = LPP; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] += __shfl_xor(o[e], off);
  }
  if (sub == 0) {
    const float inv = Lrun > 0.0f ? 1.0f / Lrun : 0.0f;
    float v[E::EPV];
    // E::store writes EPV consecutive values; stage 4 at a time
    if constexpr (E::EPV == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = o[e] * inv;
      E::store(prm.out, bh * D + dl, v);
    } else {
      // bf16: two lanes' 4 values form one 8-value store; pair lanes dl and dl + 4
      float w4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = __shfl_down(o[e], 1) * inv;
      if ((lane & 1) == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = o[e] * inv; v[4 + e] = w4[e]; }
        E::store(prm.out, bh * D + dl, v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// K3 for the append step: the merge also folds in each sequence's new token,
// read from k_new / v_new rather than the cache, and writes that token's rows
// into its slot.  The partial kernel of the same step read only the tokens
// already cached (context_lens counts them), so no kernel of the step reads a
// row written in it.  The new token is one more term of the softmax: score
// s = q . k_new in the partials' base-2 units, weight 2^(s - M), value v_new.
// ---------------------------------------------------------------------------
// Four consecutive elements as raw bits (bf16: 8 bytes in .x, .y; fp32: 16
// bytes), and the same widened to float.
template <typename E>
__device__ __forceinline__ uint4 raw4(const void* base, size_t idx) {
  if constexpr (E::EPV == 8) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    return uint4{w.x, w.y, 0u, 0u};
  } else {
    return *reinterpret_cast<const uint4*>(static_cast<const uint32_t*>(base) + idx);
  }
}

template <typename E>
__device__ __forceinline__ void widen4(const uint4& w, float (&f)[4]) {
  if constexpr (E::EPV == 8) {
    f[0] = __uint_as_float(w.x << 16);
    f[1] = __uint_as_float(w.x & 0xffff0000u);
    f[2] = __uint_as_float(w.y << 16);
    f[3] = __uint_as_float(w.y & 0xffff0000u);
  } else {
    f[0] = __uint_as_float(w.x);
    f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z);
    f[3] = __uint_as_float(w.w);
  }
}

template <typename E, int D, bool Vllm>
__global__ __launch_bounds__(64) void decode_merge_append_kernel(const DecodeParams prm, const AppendArgs ap) {
  // Lane layout as in decode_merge_kernel: lane (sub, dl) holds d = dl .. dl + 3
  // of partition rows sub, sub + PPI, ...
  constexpr int LPP = D / 4;
  constexpr int PPI = 64 / LPP;
  constexpr int KMAX = PPI * 16 <= 64 ? 16 : 64 / PPI;
  constexpr int R = PPI * KMAX;
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int KPRE = kMergeEarlyRows / PPI;
  static_assert(kMergeEarlyRows % PPI == 0 && KPRE <= KMAX, "early rows fill whole loads of round 0");
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int sub = lane / LPP;
  const int dl = (lane % LPP) * 4;
  const size_t bh = (size_t)b * prm.H + h;
  const int kvh = h / (prm.H / prm.KVH);
  const float* ml = prm.ws_ml + bh * prm.maxP * 2;
  const float* acc = prm.ws_acc + bh * prm.maxP * D;

  // Every load that needs neither the length nor the slot goes out first:
  // the new token's q, k and v (rows b of q, k_new and v_new exist whatever
  // the slot) and the first partial rows (early_rows), so the kernel makes one
  // trip to memory instead of two.  The kv head's first query head then
  // stores the new K and V rows into the slot (bit for bit), so the copy
  // drains while the partials are merged.  The partial kernel read only the
  // cached tokens, never this slot.
  const size_t row = ((size_t)b * prm.KVH + kvh) * D + dl;   // this lane's d's of k_new / v_new
  const uint4 qraw = raw4<E>(prm.q, bh * D + dl);
  const uint4 kraw = raw4<E>(ap.k_new, row);
  const uint4 vraw = raw4<E>(ap.v_new, row);
  const int early = min(prm.maxP, kMergeEarlyRows);
  f4 pre[KPRE];
  float2 mlpre;
  early_rows<D, PPI, KPRE>(acc, ml, early, sub, dl, lane, pre, mlpre);
  int n = prm.ctx[b];
  n = n < 0 ? 0 : (n > prm.max_tokens ? prm.max_tokens : n);
  const int nparts = max(1, (n + prm.P - 1) / prm.P);   // the partial kernel stored all of them
  const int64_t slot = ap.slots[b];
  const bool has_new = slot >= 0 && slot < ap.num_slots;
  if (has_new && sub == 0 && h % (prm.H / prm.KVH) == 0) {
    const size_t blk = (size_t)(slot >> prm.bs_log2);
    const size_t off = (size_t)(slot & prm.bs_mask);
    const size_t bs = (size_t)1 << prm.bs_log2;
    if constexpr (Vllm) {
      const size_t kb = (blk * prm.KVH + kvh) * D;   // element base of the (block, head) K and V blocks
      if constexpr (E::EPV == 8) {
        // K [NB, KVH, D/8, bs, 8]: d .. d + 3 lie in one 8-element group
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(ap.k_cache) + kb * bs + (size_t)(dl >> 3) * bs * 8 +
                                  off * 8 + (dl & 7)) = uint2{kraw.x, kraw.y};
        // V [NB, KVH, D, bs]: element d at column off of row d
        uint16_t* vd = static_cast<uint16_t*>(ap.v_cache) + (kb + dl) * bs + off;
        vd[0] = (uint16_t)(vraw.x & 0xffffu);
        vd[bs] = (uint16_t)(vraw.x >> 16);
        vd[2 * bs] = (uint16_t)(vraw.y & 0xffffu);
        vd[3 * bs] = (uint16_t)(vraw.y >> 16);
      } else {
        // fp32: K [NB, KVH, D/4, bs, 4]: d .. d + 3 are exactly group d / 4
        *reinterpret_cast<uint4*>(static_cast<uint32_t*>(ap.k_cache) + kb * bs + (size_t)(dl >> 2) * bs * 4 +
                                  off * 4) = kraw;
        uint32_t* vd = static_cast<uint32_t*>(ap.v_cache) + (kb + dl) * bs + off;
        vd[0] = vraw.x;
        vd[bs] = vraw.y;
        vd[2 * bs] = vraw.z;
        vd[3 * bs] = vraw.w;
      }
    } else {
      const size_t dst = (size_t)slot * prm.KVH * D + (size_t)kvh * D + dl;
      if constexpr (E::EPV == 8) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(ap.k_cache) + dst) = uint2{kraw.x, kraw.y};
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(ap.v_cache) + dst) = uint2{vraw.x, vraw.y};
      } else {
        *reinterpret_cast<uint4*>(static_cast<uint32_t*>(ap.k_cache) + dst) = kraw;
        *reinterpret_cast<uint4*>(static_cast<uint32_t*>(ap.v_cache) + dst) = vraw;
      }
    }
  }

  float Mrun = -INFINITY, Lrun = 0.0f;
  f4 o = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int r0 = 0; r0 < nparts; r0 += R) {
    const int cnt = min(R, nparts - r0);
    f4 a[KMAX];
    float2 mlv;
    round_rows<D, PPI, KMAX, KPRE>(acc, ml, r0, cnt, early, sub, dl, lane, pre, mlpre, a, mlv);
    const float M = fmaxf(Mrun, wave_max(mlv.x));
    const float w = mlv.x == -INFINITY ? 0.0f : exp2_fast(mlv.x - M);
    const float fo = Mrun == -INFINITY ? 0.0f : exp2_fast(Mrun - M);
    Lrun = Lrun * fo + wave_sum(w * mlv.y);
    o *= fo;
    Mrun = M;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) o += __shfl(w, sub + PPI * k) * a[k];
  }

  if (has_new) {
    float qf[4], kf[4], vf[4];
    widen4<E>(qraw, qf);
    widen4<E>(kraw, kf);
    widen4<E>(vraw, vf);
    float dot = qf[0] * kf[0] + qf[1] * kf[1] + qf[2] * kf[2] + qf[3] * kf[3];
#pragma unroll
    for (int off = 1; off < LPP; off <<= 1) dot += __shfl_xor(dot, off);
    // the partials' scores are (+-q or 0) . k times |scale| log2(e)
    const float sc = prm.q_mode == 2 ? 0.0f : (prm.q_mode == 1 ? -dot : dot) * prm.scale_log2;
    const float M = fmaxf(Mrun, sc);
    const float fo = Mrun == -INFINITY ? 0.0f : exp2_fast(Mrun - M);
    const float fn = exp2_fast(sc - M);
    Lrun = Lrun * fo + fn;
    o *= fo;
    if (sub == 0) o += fn * f4{vf[0], vf[1], vf[2], vf[3]};
    Mrun = M;
  }
#pragma unroll
  for (int off = LPP; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] += __shfl_xor(o[e], off);
  }
  if (sub == 0) {
    const float inv = Lrun > 0.0f ? 1.0f / Lrun : 0.0f;
    float v[E::EPV];
    if constexpr (E::EPV == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = o[e] * inv;
      E::store(prm.out, bh * D + dl, v);
    } else {
      float w4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = __shfl_down(o[e], 1) * inv;
      if ((lane & 1) == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = o[e] * inv; v[4 + e] = w4[e]; }
        E::store(prm.out, bh * D + dl, v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename E, int D, int GC, int U, int KG, int NW>
static hipError_t launch_partial_nw(const DecodeParams& prm, bool vllm, hipStream_t stream) {
  constexpr size_t kLds = NW > 1 ? (size_t)NW * 64 * GC * (E::EPV + 2) * sizeof(float) : 0;
  dim3 grid((prm.KVH / KG) * prm.nchunks, prm.maxP, prm.B);
  if (vllm) {
    if constexpr (KG == 1 && E::EPV == 4)
      hipLaunchKernelGGL((decode_partial_kernel<E, D, GC, U, KG, NW, true>), grid, dim3(64 * NW), kLds, stream, prm);
    else
      return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((decode_partial_kernel<E, D, GC, U, KG, NW>), grid, dim3(64 * NW), kLds, stream, prm);
  }
  return hipGetLastError();
}

template <typename E, int D, int GC, int U, int KG>
static hipError_t launch_partial_u(const DecodeParams& prm, int NW, bool vllm, hipStream_t stream) {
  switch (NW) {
    case 1: return launch_partial_nw<E, D, GC, U, KG, 1>(prm, vllm, stream);
    case 2: return launch_partial_nw<E, D, GC, U, KG, 2>(prm, vllm, stream);
    case 4:
      if constexpr (GC <= 4) return launch_partial_nw<E, D, GC, U, KG, 4>(prm, vllm, stream);
      break;
  }
  return hipErrorInvalidValue;
}

// (KG, U) pairs: KG kv heads per wavefront (a power of two dividing RPW),
// U loads per tile with TR * U <= block size.
template <typename E, int D, int GC, int KG>
static hipError_t launch_partial_kg(const DecodeParams& prm, const DecodePlan& plan, hipStream_t stream) {
  constexpr int RPW = 64 / (D / E::EPV);
  if constexpr (RPW % KG != 0) {
    return hipErrorInvalidValue;
  } else {
    constexpr int TR = RPW / KG;
    switch (plan.tile_unroll) {
      case 4: return launch_partial_u<E, D, GC, 4, KG>(prm, plan.waves_per_unit, plan.vllm, stream);
      case 2:
        if constexpr (TR >= 4) return launch_partial_u<E, D, GC, 2, KG>(prm, plan.waves_per_unit, plan.vllm, stream);
        break;
      case 1:
        if constexpr (TR >= 8) return launch_partial_u<E, D, GC, 1, KG>(prm, plan.waves_per_unit, plan.vllm, stream);
        break;
    }
    return hipErrorInvalidValue;
  }
}

template <typename E, int D, int GC>
static hipError_t launch_partial_gc(const DecodeParams& prm, const DecodePlan& plan, hipStream_t s) {
  switch (plan.kv_per_wave) {
    case 1: return launch_partial_kg<E, D, GC, 1>(prm, plan, s);
    case 2: return launch_partial_kg<E, D, GC, 2>(prm, plan, s);
    case 4: return launch_partial_kg<E, D, GC, 4>(prm, plan, s);
    case 8: return launch_partial_kg<E, D, GC, 8>(prm, plan, s);
  }
  return hipErrorInvalidValue;
}

template <typename E, int D>
static hipError_t launch_partial_d(const DecodeParams& prm, const DecodePlan& plan, hipStream_t s) {
  switch (plan.heads_per_unit) {
    case 1: return launch_partial_gc<E, D, 1>(prm, plan, s);
    case 2: return launch_partial_gc<E, D, 2>(prm, plan, s);
    case 4: return launch_partial_gc<E, D, 4>(prm, plan, s);
    case 8: return launch_partial_gc<E, D, 8>(prm, plan, s);
  }
  return hipErrorInvalidValue;
}

template <typename E>
static hipError_t launch_partial_e(const DecodeParams& prm, int32_t D, const DecodePlan& plan,
                                   hipStream_t s) {
  switch (D) {
    case 64: return launch_partial_d<E, 64>(prm, plan, s);
    case 128: return launch_partial_d<E, 128>(prm, plan, s);
    case 256: return launch_partial_d<E, 256>(prm, plan, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_partials(const DecodeParams& prm, int32_t dtype, int32_t D,
                                  const DecodePlan& plan, hipStream_t stream) {
  return dtype == 0 ? launch_partial_e<F32>(prm, D, plan, stream)
                    : launch_partial_e<BF16>(prm, D, plan, stream);
}

template <typename E>
static hipError_t launch_merge_e(const DecodeParams& prm, int32_t D, hipStream_t stream) {
  const dim3 grid(prm.H, prm.B);
  const size_t lds = 0;
  switch (D) {
    case 64: hipLaunchKernelGGL((decode_merge_kernel<E, 64>), grid, dim3(64), lds, stream, prm); break;
    case 128: hipLaunchKernelGGL((decode_merge_kernel<E, 128>), grid, dim3(64), lds, stream, prm); break;
    case 256: hipLaunchKernelGGL((decode_merge_kernel<E, 256>), grid, dim3(64), lds, stream, prm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeParams& prm, int32_t dtype, int32_t D,
                               hipStream_t stream) {
  return dtype == 0 ? launch_merge_e<F32>(prm, D, stream) : launch_merge_e<BF16>(prm, D, stream);
}

template <typename E, bool Vllm>
static hipError_t launch_merge_append_e(const DecodeParams& prm, const AppendArgs& ap, int32_t D,
                                        hipStream_t stream) {
  const dim3 grid(prm.H, prm.B);
  switch (D) {
    case 64: hipLaunchKernelGGL((decode_merge_append_kernel<E, 64, Vllm>), grid, dim3(64), 0, stream, prm, ap); break;
    case 128: hipLaunchKernelGGL((decode_merge_append_kernel<E, 128, Vllm>), grid, dim3(64), 0, stream, prm, ap); break;
    case 256: hipLaunchKernelGGL((decode_merge_append_kernel<E, 256, Vllm>), grid, dim3(64), 0, stream, prm, ap); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_merge_append(const DecodeParams& prm, const AppendArgs& ap, int32_t dtype, int32_t D,
                                      hipStream_t stream) {
  if (dtype == 0) return ap.vllm ? launch_merge_append_e<F32, true>(prm, ap, D, stream)
                                 : launch_merge_append_e<F32, false>(prm, ap, D, stream);
  return ap.vllm ? launch_merge_append_e<BF16, true>(prm, ap, D, stream)
                 : launch_merge_append_e<BF16, false>(prm, ap, D, stream);
}

}  // namespace pa
