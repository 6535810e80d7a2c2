// Tile helpers shared by the bf16 matrix-core kernels (paged decode in
// pa_decode_mfma.hip, paged prefill in pa_prefill.hip): 16-byte buffer loads
// of 16-token tiles of one kv head through the block table, their swizzled
// LDS layout, the per-lane LDS addresses of the K and transposed V operands,
// and the cross-lane reductions of the 16x16 accumulator layout.
// Operand layouts (v_mfma_f32_16x16x32_bf16): A lane l holds row l % 16,
// k = 8 (l / 16) .. + 7; B lane l holds column l % 16, the same k; the
// 16x16 fp32 accumulator gives lane l column l % 16, rows 4 (l / 16) + i.
#pragma once

#include <math.h>

#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4m __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3M = 0x00020000;   // raw untyped buffer access, gfx9 family
constexpr float kSlackM = 8.0f;           // lazy-rescale slack (base-2 units)

__device__ __forceinline__ float exp2m(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum over the four 16-lane groups (lanes xor 16, xor 32)
__device__ __forceinline__ float groups_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float groups_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// LDS slot swizzle: 16-byte piece pc of token row t is stored at piece
// pc ^ swz(t) of the row (a bijection within the row for any swz, so writes
// and reads only have to agree).  It is chosen from the bank behaviour
// measured on gfx950 with a probe of each access pattern (SQ_LDS_IDX_ACTIVE
// and SQ_LDS_BANK_CONFLICT per instruction): 64 banks of 4 bytes; a 16-byte
// read is served 16 consecutive lanes per cycle (4 cycles per instruction
// at best), an 8-byte transposing read 32 lanes per cycle (2 at best); and
// address bit 11 flips bit 2 of the bank index.  That model predicted all 36
// probe measurements.  Under it:
// - head_dim 128 (16 pieces per row): the K operand reads (16 rows, one piece
//   each, lanes of one 16-lane group) need swz(t) ^ (t >> 3) to be a
//   permutation, and the transposed V reads (8 rows per 32 lanes, a 32-byte
//   piece pair each) need swz(t) >> 1 distinct over each 8 rows.
//   swz(t) = (t mod 8) * 2 does both, at any base address: 4 and 2 cycles
//   per instruction, against 8 and 2 for the previous choice
//   ((t mod 8) * 2 + t / 8), which the bank hash folded onto itself.
// - head_dim 256 (32 pieces): ((t mod 8) * 2 + t / 8) is conflict-free for
//   both reads at any base.
// - head_dim 64 (8 pieces): u ^ (u mod 2) * 4 with u = t / 2 makes the V
//   reads conflict-free at any base and the K reads too at 2 KiB-aligned
//   tiles (t / 2 before: V reads at twice their cycles).
// The tile writes (ds_write_b128, 4 rows of whole pieces per instruction) are
// conflict-free under every swizzle tried.
template <int PPR>
__device__ __forceinline__ int swz(int t) {
  if constexpr (PPR >= 32) {
    return ((t & 7) << 1) | (t >> 3);
  } else if constexpr (PPR == 16) {
    return (t & 7) << 1;
  } else {
    const int u = t >> 1;
    return u ^ ((u & 1) << 2);
  }
}

template <int D>
struct Geo {
  static constexpr int ROWB = D * 2;        // bytes of one (token, kv head) row
  static constexpr int PPR = ROWB / 16;     // 16-byte pieces per row
  static constexpr int TPI = 64 / PPR;      // token rows per load instruction
  static constexpr int NI = 16 / TPI;       // load instructions per 16-token tile (K, and again V)
  static constexpr int NQK = D / 32;        // QK products (32 d each)
  static constexpr int NPV = D / 16;        // PV products (16 d columns each)
};

// The kv head's column of the caches.
template <int D>
__device__ __forceinline__ const char* kv_col(const void* cache, int kvh) {
  return static_cast<const char*>(cache) + (size_t)kvh * Geo<D>::ROWB;
}

template <int A>
struct CachePolicy {
  static constexpr int aux = A;
};
constexpr int kAuxNT = 2;   // buffer-load cache policy bit "nt": non-temporal (streaming) access

// Loads of the 16-token tile starting at token `tile` of a partition ending
// at t_end: instruction u brings token rows u * TPI + lane / PPR, piece
// lane % PPR, of the kv head (kc, vc: the kv head's column of the caches).
// ph0 is the physical block holding the tile's first token, ph1 (blocks of 8
// tokens only) the next one.  A buffer resource starts at the first row it
// covers and ends after the last valid row of the partition, so rows past the
// end (and blocks outside the pool, and every row of a dead load) read zeros.
// AUX is the loads' cache policy: kAuxNT when the rows are read once in this
// call, 0 (default) when other sequences are likely to read the same blocks
// (a shared prefix).
// Returns the tile's row validity mask (bit r: row r holds a token).
// WholeTile: block_size >= 16, so a tile (tiles start at multiples of 16,
// partitions at multiples of the block size) lies inside one block;
// otherwise the block size is 8 and a tile spans two blocks.
template <int D, bool WholeTile, int AUX, class Prm>
__device__ __forceinline__ uint32_t load_tile(const Prm& prm, const char* kc, const char* vc, int t_end,
                                              int tile, bool live, int ph0, int ph1, uint32_t lane_off,
                                              u32x4m (&kr)[Geo<D>::NI], u32x4m (&vr)[Geo<D>::NI]) {
  constexpr int TPI = Geo<D>::TPI, NI = Geo<D>::NI;
  const uint32_t row_bytes = (uint32_t)prm.KVH * Geo<D>::ROWB;
  const size_t blk_bytes = (size_t)row_bytes << prm.bs_log2;
  uint32_t ok = 0;
  if constexpr (WholeTile) {
    const int nv = min(16, t_end - tile);               // valid rows of the tile
    const bool good = live && (unsigned)ph0 < (unsigned)prm.NB && nv > 0;
    const size_t off = (size_t)(good ? ph0 : 0) * blk_bytes + (size_t)(tile & prm.bs_mask) * row_bytes;
    const int nrec = good ? nv * (int)row_bytes : 0;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + off), (short)0, nrec, kRsrcWord3M);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + off), (short)0, nrec, kRsrcWord3M);
#pragma unroll
    for (int u = 0; u < NI; ++u) kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off, u * TPI * row_bytes, AUX);
#pragma unroll
    for (int u = 0; u < NI; ++u) vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off, u * TPI * row_bytes, AUX);
    if (good) ok = nv >= 16 ? 0xffffu : ((1u << nv) - 1u);
  } else {
    // One resource per instruction; instructions 0 .. NI/2-1 read block ph0
    // (tokens tile .. tile+7), the others block ph1.
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int t0 = tile + u * TPI;                   // first token of this instruction
      const int phys = u * TPI >= 8 ? ph1 : ph0;
      const int nv = min(TPI, t_end - t0);             // valid rows of this instruction
      const bool good = live && (unsigned)phys < (unsigned)prm.NB && nv > 0;
      const size_t off = (size_t)(good ? phys : 0) * blk_bytes + (size_t)(t0 & prm.bs_mask) * row_bytes;
      const int nrec = good ? nv * (int)row_bytes : 0;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + off), (short)0, nrec, kRsrcWord3M);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + off), (short)0, nrec, kRsrcWord3M);
      kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off, 0, AUX);
      vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off, 0, AUX);
      if (good) ok |= ((1u << nv) - 1u) << (u * TPI);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  return ok;
}

// Per-lane LDS addresses: where the tile's loads are written, and where the
// K operand (row tk) and the transposed V operand (rows tv.., d offset dv)
// are read.
template <int D>
struct LdsMap {
  int wr[Geo<D>::NI];
  int tk, tv, dv;
  __device__ __forceinline__ explicit LdsMap(int lane) {
    constexpr int PPR = Geo<D>::PPR, TPI = Geo<D>::TPI;
#pragma unroll
    for (int u = 0; u < Geo<D>::NI; ++u) {
      const int t = u * TPI + lane / PPR, pc = lane % PPR;
      wr[u] = (t * PPR + (pc ^ swz<PPR>(t))) * 16;
    }
    tk = lane & 15;
    tv = 4 * (lane >> 4) + ((lane & 15) >> 2);
    dv = 4 * (lane & 3);
  }
};

}  // namespace pa
