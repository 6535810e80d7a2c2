// Paged decode attention for gfx950, bf16 caches: split-KV partial kernel on
// the matrix cores.
//
// Same operation and partial-result format as decode_partial_kernel in
// pa_decode.hip ("P09 · Paged KV 写入 + decode attention", 题面速览 and the decode
// shape trace; online softmax over the block table as on "PagedAttention
// kernel：paged KV cache 与 block table", 直接答案 and 深入原理 for the split),
// for the layouts where both products are dense contractions worth the matrix
// cores: every 16-token tile of one kv head gives
//   S   = K_tile (16 x D) . Q^T (D x 16 query-head columns)   v_mfma_f32_16x16x32_bf16
//   O^T += V_tile^T (D x 16) . P^T (16 x 16)                   v_mfma_f32_16x16x16_bf16
// with up to 16 query heads of the kv head's GQA group as the 16 columns.
//
// Data movement per tile: 16-byte buffer loads (coalesced runs of whole
// D-rows, double buffered in registers) are written to LDS in a swizzled
// order, then read back in operand order: K with ds_read_b128, V with the
// transposing ds_read_b64_tr_b16, which hands each lane four tokens of one
// d-column.  The accumulator layout of S (lane: head = lane % 16, tokens
// 4 * (lane / 16) + i) is the operand layout P^T needs, so the probabilities
// never leave the lane that computed them, and O^T (lane: head = lane % 16,
// d = 16 n + 4 * (lane / 16) + i) shares that head-per-lane layout, so the
// softmax rescaling and the final division are per-lane.
//
// The scores are exact products of bf16 values summed in fp32; the
// probabilities enter the PV product rounded to bf16 (the running sums l use
// the unrounded fp32 values).
#include <math.h>

#include "pa_internal.h"

namespace pa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4m __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3M = 0x00020000;   // raw untyped buffer access, gfx9 family
constexpr float kSlackM = 8.0f;           // lazy-rescale slack (base-2 units)
constexpr int kPersistentWavesPerCU = 8;  // resident workgroups (one wavefront each) per CU

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
// pc ^ sw(t) of the row.  sw is a permutation of the 16 rows' residues so that
// the K operand reads (16 rows, one piece each) and the transposed V reads
// (4 rows, two adjacent pieces each) fall in distinct bank groups.
template <int PPR>
__device__ __forceinline__ int swz(int t) {
  if constexpr (PPR >= 16)
    return ((t & 7) << 1) | (t >> 3);
  else
    return t >> 1;
}

}  // namespace

// One work unit: partition p of sequence b, kv head kvh, query-head chunk
// chunk (up to 16 heads of the kv head's group).  WholeTile: block_size >= 16,
// so every 16-token tile (tiles start at multiples of 16 and partitions at
// multiples of the block size) lies inside one block.
template <int D, bool WholeTile>
__device__ __forceinline__ void mfma_unit(const DecodeParams& prm, int b, int p, int kvh, int chunk,
                                          uint8_t* __restrict__ lds_k, uint8_t* __restrict__ lds_v) {
  constexpr int ROWB = D * 2;        // bytes of one (token, kv head) row
  constexpr int PPR = ROWB / 16;     // 16-byte pieces per row
  constexpr int TPI = 64 / PPR;      // token rows per load instruction
  constexpr int NI = 16 / TPI;       // load instructions per 16-token tile (K, and again V)
  constexpr int NQK = D / 32;        // QK products (32 d each)
  constexpr int NPV = D / 16;        // PV products (16 d columns each)

  const int G = prm.H / prm.KVH;
  const int h_base = kvh * G + chunk * 16;
  const int nh = min(16, G - chunk * 16);

  int n = prm.ctx[b];
  n = n < 0 ? 0 : (n > prm.max_tokens ? prm.max_tokens : n);
  const int nparts = (n + prm.P - 1) / prm.P;
  if (p >= (nparts > 0 ? nparts : 1)) return;
  const int t_begin = p * prm.P;
  const int t_end = min(n, t_begin + prm.P);

  const int lane = threadIdx.x;
  const int col = lane & 15;         // query head (column) of this lane
  const int grp = lane >> 4;         // 16-lane group
  const bool head_ok = col < nh;

  // Q^T operands: lane holds q[head col][32 c + 8 grp .. + 8] (zero for padding
  // columns).  A negative scale is applied as negated q, a zero scale as zero q.
  bf16x8 qop[NQK];
  {
    const uint32_t flip = prm.q_mode == 1 ? 0x80008000u : 0u;
    const uint32_t keep = (prm.q_mode == 2 || !head_ok) ? 0u : 0xffffffffu;
    const uint8_t* qrow = static_cast<const uint8_t*>(prm.q) +
                          ((size_t)(b * prm.H + h_base + (head_ok ? col : 0)) * D) * 2;
#pragma unroll
    for (int c = 0; c < NQK; ++c) {
      u32x4m w = *reinterpret_cast<const u32x4m*>(qrow + (32 * c + 8 * grp) * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t x = w[i];
        w[i] = (x ^ flip) & keep;
      }
      qop[c] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const float cs = prm.scale_log2;

  // Softmax state of column col (uniform over the four groups), this lane's
  // share of the running sum, and O^T accumulators.
  float m = -INFINITY, mneg = 0.0f, lsum = 0.0f;
  f32x4 o[NPV];
#pragma unroll
  for (int j = 0; j < NPV; ++j) o[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const uint32_t row_bytes = (uint32_t)prm.KVH * ROWB;
  const size_t blk_bytes = (size_t)row_bytes << prm.bs_log2;
  const char* kc = static_cast<const char*>(prm.k_cache) + (size_t)kvh * ROWB;
  const char* vc = static_cast<const char*>(prm.v_cache) + (size_t)kvh * ROWB;
  const int32_t* tbl = prm.tables + (size_t)b * prm.W;
  const int j_first = t_begin >> prm.bs_log2;
  const int j_end = (t_end + prm.bs_mask) >> prm.bs_log2;
  const int tbl_v = (j_first + lane < j_end) ? tbl[j_first + lane] : 0;

  // Loads: instruction u of a tile brings token rows u * TPI + lane / PPR,
  // piece lane % PPR, of the kv head.  Its buffer resource starts at the
  // first row it covers and ends after the last valid row of the sequence, so
  // rows past the end (and blocks outside the pool) read zeros.
  const uint32_t lane_off = (uint32_t)(lane / PPR) * row_bytes + (uint32_t)(lane % PPR) * 16;
  // LDS byte address each lane writes for instruction u, and reads for the K
  // operand of product c / the V operand of product j.
  int wr_addr[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int t = u * TPI + lane / PPR, pc = lane % PPR;
    wr_addr[u] = (t * PPR + (pc ^ swz<PPR>(t))) * 16;
  }
  const int tk = col;                                // K operand row (token) of this lane
  const int tv = 4 * grp + ((lane & 15) >> 2);       // V rows read by this lane (tr layout)
  const int dv = 4 * (lane & 3);                     // d offset within a 16-column chunk

  u32x4m kA[NI], vA[NI], kB[NI], vB[NI];
  uint32_t okA = 0, okB = 0;                         // per-row validity mask of the tile (bit r)

  auto load_tile = [&](int tile, u32x4m (&kr)[NI], u32x4m (&vr)[NI]) -> uint32_t {
    uint32_t ok = 0;
    if constexpr (WholeTile) {
      // The 16 rows lie in one block: one resource per tile, instruction u at
      // a scalar offset of u * TPI rows.
      const int phys = __builtin_amdgcn_readlane(tbl_v, (tile >> prm.bs_log2) - j_first);
      const int nv = min(16, t_end - tile);             // valid rows of the tile
      const bool good = (unsigned)phys < (unsigned)prm.NB && nv > 0;
      const size_t off = (size_t)(good ? phys : 0) * blk_bytes + (size_t)(tile & prm.bs_mask) * row_bytes;
      const int nrec = good ? nv * (int)row_bytes : 0;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + off), (short)0, nrec, kRsrcWord3M);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + off), (short)0, nrec, kRsrcWord3M);
#pragma unroll
      for (int u = 0; u < NI; ++u) kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off, u * TPI * row_bytes, 0);
#pragma unroll
      for (int u = 0; u < NI; ++u) vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off, u * TPI * row_bytes, 0);
      if (good) ok = nv >= 16 ? 0xffffu : ((1u << nv) - 1u);
    } else {
      // Blocks shorter than a tile: one resource per instruction.
#pragma unroll
      for (int u = 0; u < NI; ++u) {
        const int t0 = tile + u * TPI;                   // first token of this instruction
        const int phys = __builtin_amdgcn_readlane(tbl_v, (t0 >> prm.bs_log2) - j_first);
        const int nv = min(TPI, t_end - t0);             // valid rows of this instruction
        const bool good = (unsigned)phys < (unsigned)prm.NB && nv > 0;
        const size_t off = (size_t)(good ? phys : 0) * blk_bytes + (size_t)(t0 & prm.bs_mask) * row_bytes;
        const int nrec = good ? nv * (int)row_bytes : 0;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kc + off), (short)0, nrec, kRsrcWord3M);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vc + off), (short)0, nrec, kRsrcWord3M);
        kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off, 0, 0);
        vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off, 0, 0);
        if (good) ok |= ((1u << nv) - 1u) << (u * TPI);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    return ok;
  };

  auto fold_tile = [&](uint32_t ok, const u32x4m (&kr)[NI], const u32x4m (&vr)[NI]) {
    // Stage the tile in LDS (the previous tile's reads were issued earlier by
    // this wavefront, and LDS serves one wavefront's accesses in order).
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      *reinterpret_cast<u32x4m*>(lds_k + wr_addr[u]) = kr[u];
      *reinterpret_cast<u32x4m*>(lds_v + wr_addr[u]) = vr[u];
    }
    // S = K_tile . Q^T: lane holds S[token 4 grp + i][head col].
    f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < NQK; ++c) {
      const int pc = 4 * c + grp;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds_k + (tk * PPR + (pc ^ swz<PPR>(tk))) * 16);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[c], s, 0, 0, 0);
    }
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = (ok >> (4 * grp + i)) & 1u;
      sc[i] = valid ? s[i] * cs : -INFINITY;
    }
    float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mt = groups_max(mt);
    if (__builtin_amdgcn_ballot_w64(mt > m + kSlackM)) {   // wavefront-uniform, rare
      if (mt > m) {
        const float corr = exp2m(m - mt);                  // 0 while m is -inf
        m = mt;
        mneg = -mt;
        lsum *= corr;
#pragma unroll
        for (int j = 0; j < NPV; ++j) o[j] *= corr;
      }
    }
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = exp2m(sc[i] + mneg);
      lsum += pr[i];
    }
    bf16x4 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[i] = (__bf16)pr[i];
    // O^T += V_tile^T . P^T, one 16-column d chunk per product.
#pragma unroll
    for (int j = 0; j < NPV; ++j) {
      const int d = 16 * j + dv;
      const int pc = d >> 3;
      const int addr = (tv * PPR + (pc ^ swz<PPR>(tv))) * 16 + (d & 7) * 2;
      const s16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(lds_v + addr));
      o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, vt), pb, o[j], 0, 0, 0);
    }
  };

  const int ntok = t_end - t_begin;
  const int ntiles = ntok > 0 ? (ntok + 15) / 16 : 0;
  if (ntiles > 0) {
    auto tile_at = [&](int i) { return t_begin + min(i, ntiles - 1) * 16; };
    okA = load_tile(tile_at(0), kA, vA);
    const int npairs = ntiles >> 1;
    for (int ip = 0; ip < npairs; ++ip) {
      okB = load_tile(tile_at(2 * ip + 1), kB, vB);
      fold_tile(okA, kA, vA);
      okA = load_tile(tile_at(2 * ip + 2), kA, vA);
      fold_tile(okB, kB, vB);
    }
    if (ntiles & 1) fold_tile(okA, kA, vA);
  }

  // Column col's totals.
  const float L = groups_sum(lsum);
  const size_t bh = (size_t)b * prm.H + h_base + col;
  auto store_out = [&](const f32x4 (&acc)[NPV], float inv) {
    uint16_t* outp = static_cast<uint16_t*>(prm.out) + bh * D;
#pragma unroll
    for (int j = 0; j < NPV; ++j) {
      bf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (__bf16)(acc[j][i] * inv);
      *reinterpret_cast<bf16x4*>(outp + 16 * j + 4 * grp) = w;
    }
  };
  if (nparts <= 1) {
    if (head_ok) store_out(o, L > 0.0f ? 1.0f / L : 0.0f);
    return;
  }
  // Partial results (fp32) for the merge kernel.
  if (head_ok) {
    const size_t slot = bh * prm.maxP + p;
    float* dst = prm.ws_acc + slot * D;
#pragma unroll
    for (int j = 0; j < NPV; ++j) *reinterpret_cast<f32x4*>(dst + 16 * j + 4 * grp) = o[j];
    if (grp == 0) *reinterpret_cast<float2*>(prm.ws_ml + slot * 2) = make_float2(m, L);
  }
}

// Grid form (sequence counts beyond the persistent form's search): one
// workgroup per unit.  Grid x = (kv head, head chunk) fastest, y = partition,
// z = sequence; units past a sequence's last partition exit at once.
template <int D, bool WholeTile>
__global__ __launch_bounds__(64) void decode_partial_mfma_grid_kernel(const DecodeParams prm) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[16 * 2 * D];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[16 * 2 * D];
  const int kvh = blockIdx.x / prm.nchunks;
  mfma_unit<D, WholeTile>(prm, blockIdx.z, blockIdx.y, kvh, blockIdx.x - kvh * prm.nchunks, lds_k, lds_v);
}

// Persistent form: as many workgroups as stay resident (a fixed number per
// CU) walk a list of the units that exist, so that the chip holds its full
// complement of wavefronts from the first tile to the drain, with no
// workgroup dispatch between units and no empty units.
//
// The list: first every sequence's partitions before its last one (all full,
// P tokens), sequence by sequence, then the last partition of each sequence;
// each (sequence, partition) pair expands into kv heads x head chunks
// consecutive units.  Round r of the walk hands units r*G .. r*G + G-1 to the
// G workgroups, in forward order on even rounds and reverse order on odd
// ones, so that a workgroup that drew a late (short) unit in one round draws
// an early one in the next.  The list is rebuilt by every workgroup from the
// context lengths (an exclusive scan into LDS), so all of them agree on it
// without any communication.
template <int D, bool WholeTile>
__global__ __launch_bounds__(64) void decode_partial_mfma_kernel(const DecodeParams prm) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[16 * 2 * D];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[16 * 2 * D];
  extern __shared__ int32_t s_first[];          // [B]: list index of sequence b's first full pair
  const int lane = threadIdx.x;
  const int B = prm.B, P = prm.P;
  auto nparts_of = [&](int b) {
    int n = prm.ctx[b];
    n = n < 0 ? 0 : (n > prm.max_tokens ? prm.max_tokens : n);
    return (n + P - 1) / P;
  };
  int carry = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    int f = 0;
    if (b < B) {
      const int np = nparts_of(b);
      f = np > 1 ? np - 1 : 0;
    }
    int incl = f;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    if (b < B) s_first[b] = carry + incl - f;
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  __syncthreads();
  const uint32_t F = (uint32_t)carry;           // pairs of full partitions
  const uint32_t upp = (uint32_t)(prm.KVH * prm.nchunks);
  const uint32_t nunits = (F + (uint32_t)B) * upp;
  const uint32_t G = gridDim.x;
  const int stride = (B + 63) >> 6;             // sequences per lane in the first search level

  uint32_t t = blockIdx.x;
  for (uint32_t round = 1; t < nunits; ++round) {
    const uint32_t pair = t / upp, sub = t - pair * upp;
    int b, p;
    if (pair < F) {
      // b = the last sequence whose first list index is <= pair: one ballot
      // over every stride-th sequence, then one inside the chosen stretch
      const int i1 = lane * stride;
      const uint64_t m1 = __ballot(i1 < B && (uint32_t)s_first[i1 < B ? i1 : 0] <= pair);
      const int seg = __popcll(m1) - 1;
      const int i2 = seg * stride + lane;
      const uint64_t m2 = __ballot(lane < stride && i2 < B && (uint32_t)s_first[i2 < B ? i2 : 0] <= pair);
      b = __builtin_amdgcn_readfirstlane(seg * stride + __popcll(m2) - 1);
      p = (int)(pair - (uint32_t)s_first[b]);
    } else {
      b = (int)(pair - F);
      const int np = nparts_of(b);
      p = np > 0 ? np - 1 : 0;
    }
    const int kvh = (int)(sub / (uint32_t)prm.nchunks);
    mfma_unit<D, WholeTile>(prm, b, p, kvh, (int)sub - kvh * prm.nchunks, lds_k, lds_v);
    t = round * G + ((round & 1) ? G - 1 - blockIdx.x : blockIdx.x);
  }
}

namespace {
constexpr int kMaxPersistentSeqs = 4096;   // the pair search covers 64 x 64 sequences

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

template <int D, bool WholeTile>
hipError_t launch_mfma(const DecodeParams& prm, hipStream_t stream) {
  if (prm.B <= kMaxPersistentSeqs) {
    const size_t lds = (size_t)prm.B * sizeof(int32_t);
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void*>(&decode_partial_mfma_kernel<D, WholeTile>), 64, lds);
    const int cus = device_cus();
    if (e == hipSuccess && per_cu > 0 && cus > 0) {
      if (per_cu > kPersistentWavesPerCU) per_cu = kPersistentWavesPerCU;
      const int64_t units_max = (int64_t)prm.B * prm.maxP * prm.KVH * prm.nchunks;
      const int64_t wgs = (int64_t)per_cu * cus < units_max ? (int64_t)per_cu * cus : units_max;
      hipLaunchKernelGGL((decode_partial_mfma_kernel<D, WholeTile>), dim3((uint32_t)wgs), dim3(64), lds, stream,
                         prm);
      return hipGetLastError();
    }
  }
  const dim3 grid(prm.KVH * prm.nchunks, prm.maxP, prm.B);
  hipLaunchKernelGGL((decode_partial_mfma_grid_kernel<D, WholeTile>), grid, dim3(64), 0, stream, prm);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_partials_mfma(const DecodeParams& prm, int32_t D, hipStream_t stream) {
  const bool whole = prm.bs_log2 >= 4;
  switch (D) {
    case 64: return whole ? launch_mfma<64, true>(prm, stream) : launch_mfma<64, false>(prm, stream);
    case 128: return whole ? launch_mfma<128, true>(prm, stream) : launch_mfma<128, false>(prm, stream);
    case 256: return whole ? launch_mfma<256, true>(prm, stream) : launch_mfma<256, false>(prm, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
