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
//   O^T += V_tile^T (D x 16) . P^T (16 x 16)                   v_mfma_f32_16x16x32_bf16
//                                    (P as hi + lo, V twice along the contraction)
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
// probabilities enter the PV product as a pair of bf16 values whose sum is
// the fp32 probability to about 2^-17 relative (split_bf16), and the running
// sums l add the fp32 values, so the weighted sum is fp32 softmax . V.
#include <math.h>

#include "pa_mfma_tile.h"

#ifdef PA_TIMELINE
// Timeline build only (compiled with -DPA_TIMELINE into a separate library;
// the library proper contains none of this).  The persistent kernel records
// per wavefront its s_memrealtime stamps (100 MHz) at entry, when the unit
// list is ready and at exit, with its hardware ids; and per unit its
// description with the stamps of its start and end.  Lane 0 writes them with
// vector stores; pa_timeline_read copies the buffer to the host.
// Layout (64-bit words): [0] units recorded; [16 + 4 w ..) wavefront w =
// workgroup * NW + wave; [kTlUnitBase + 4 u ..) unit record u.
#include "../../include/paged_kv.h"
namespace pa {
constexpr int kTlWords = 1 << 16, kTlUnitBase = 32768, kTlMaxUnits = 8000;
__device__ uint64_t g_timeline[kTlWords];
}  // namespace pa
extern "C" int pa_timeline_read(void* dst, size_t bytes) {
  if (!dst || bytes > sizeof(uint64_t) * pa::kTlWords) return PA_ERR_SHAPE;
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(pa::g_timeline), bytes, 0, hipMemcpyDeviceToHost) == hipSuccess
             ? PA_OK : PA_ERR_LAUNCH;
}
extern "C" int pa_timeline_reset() {
  static uint64_t zero[pa::kTlWords];
  return hipMemcpyToSymbol(HIP_SYMBOL(pa::g_timeline), zero, sizeof(zero), 0, hipMemcpyHostToDevice) == hipSuccess
             ? PA_OK : PA_ERR_LAUNCH;
}
#endif

namespace pa {

namespace {

constexpr int kBuckets = 64;              // length classes of the last-partition ordering

// One work unit: partition p of sequence b (n tokens, np partitions), kv head
// kvh, query-head chunk chunk (up to 16 heads of the kv head's group), tokens
// [t_begin, t_end) in ntiles tiles of TOK tokens (16; 32 for vLLM's layout
// with blocks of 32 tokens or more) (at least one: an empty unit folds one
// fully masked tile and writes zeros).  Wave-uniform.
// A shared unit (ns > 0) folds a shared partition p for ns sequences at once:
// entries g0 .. g0 + ns - 1 of the list of sequences that share the prefix,
// their G heads side by side as the 16 columns; b is the first of them (whose
// table row, equal to theirs over the prefix, gives the blocks).
struct Unit {
  int b, p, kvh, chunk, np;
  int t_begin, t_end, ntiles;
  int ns, g0;
};

template <int TOK = 16>
__device__ __forceinline__ Unit make_unit(const DecodeParams& prm, int b, int p, int n, int kvh, int chunk) {
  Unit u;
  u.b = b;
  u.p = p;
  u.kvh = kvh;
  u.chunk = chunk;
  u.np = (n + prm.P - 1) / prm.P;
  u.t_begin = p * prm.P;
  u.t_end = min(n, u.t_begin + prm.P);
  const int ntok = u.t_end - u.t_begin;
  u.ntiles = ntok > 0 ? (ntok + TOK - 1) / TOK : 1;
  u.ns = 0;
  u.g0 = 0;
  return u;
}

// Sequence and query head of product column col (lane % 16) of a unit: the
// unit's sequence and head chunk col, or for a shared unit sequence col / G
// of its group and head col % G.  Padding columns map to the unit's first
// sequence and head (masked later).  jn: the shared-prefix sequence list
// (read only for shared units, which only the persistent form folds:
// Shared = false compiles them out).
struct ColHead {
  int b, h;
  bool ok;
};
template <bool Shared>
__device__ __forceinline__ ColHead column_head(const DecodeParams& prm, const Unit& u, int col,
                                               const int32_t* jn) {
  const int G = prm.H / prm.KVH;
  ColHead c;
  if (Shared && u.ns > 0) {
    const int j = col / G;
    c.ok = j < u.ns;
    // padding columns read the group's first member (u.b) from the list too:
    // a choice between the list and u.b becomes a load through a selected
    // address, which keeps the unit in scratch memory
    c.b = jn[u.g0 + (c.ok ? j : 0)];
    c.h = u.kvh * G + (c.ok ? col - j * G : 0);
  } else {
    const int nh = min(16, G - u.chunk * 16);
    c.ok = col < nh;
    c.b = u.b;
    c.h = u.kvh * G + u.chunk * 16 + (c.ok ? col : 0);
  }
  return c;
}

// The neighbour sequence of b (the previous one, or sequence 1 for sequence
// 0): sequences that share a prefix usually sit next to each other in a
// batch (samples of one prompt), or all share it (a common system prompt).
__device__ __forceinline__ int neighbour(const DecodeParams& prm, int b) {
  return b > 0 ? b - 1 : (prm.B > 1 ? 1 : -1);
}

// Inclusive prefix sum over the 64 lanes of a wavefront with data-parallel
// moves (no LDS round trips): row shifts by 1, 2, 4 and 8 scan each row of 16
// lanes, then lane 15's sum is broadcast into rows 1 and 3 and lane 31's into
// rows 2 and 3.  Lanes a move leaves out keep 0.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}

__device__ __forceinline__ int clamp_len(const DecodeParams& prm, int n) {
  return n < 0 ? 0 : (n > prm.max_tokens ? prm.max_tokens : n);
}

// Raw Q^T operands of a unit: lane holds q[head col][32 c + 8 grp .. + 8] of
// its column's head (head 0 of the chunk for padding columns, masked later).
template <int D, bool Shared = false>
__device__ __forceinline__ void load_q(const DecodeParams& prm, const Unit& u, int lane,
                                       u32x4m (&qr)[Geo<D>::NQK], const int32_t* jn) {
  const int grp = lane >> 4;
  const ColHead c = column_head<Shared>(prm, u, lane & 15, jn);
  const uint8_t* qrow = static_cast<const uint8_t*>(prm.q) + ((size_t)((size_t)c.b * prm.H + c.h) * D) * 2;
#pragma unroll
  for (int c = 0; c < Geo<D>::NQK; ++c)
    qr[c] = *reinterpret_cast<const u32x4m*>(qrow + (32 * c + 8 * grp) * 2);
}

// Q^T operands from the raw loads: zero for padding columns; a negative scale
// is applied as negated q, a zero scale as zero q.
template <int D>
__device__ __forceinline__ void q_operands(const DecodeParams& prm, const Unit& u, int lane,
                                           const u32x4m (&qr)[Geo<D>::NQK], bf16x8 (&qop)[Geo<D>::NQK]) {
  const int G = prm.H / prm.KVH;
  const int col = lane & 15;
  const bool head_ok = u.ns > 0 ? col / G < u.ns : col < min(16, G - u.chunk * 16);
  const uint32_t flip = prm.q_mode == 1 ? 0x80008000u : 0u;
  const uint32_t keep = (prm.q_mode == 2 || !head_ok) ? 0u : 0xffffffffu;
#pragma unroll
  for (int c = 0; c < Geo<D>::NQK; ++c) {
    u32x4m w = qr[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = w[i];
      w[i] = (x ^ flip) & keep;
    }
    qop[c] = __builtin_bit_cast(bf16x8, w);
  }
}

// Probabilities as the B operand of the P.V products, carried exactly enough
// for fp32: p = hi + lo with hi = bf16(p) (round to nearest even) and
// lo = bf16(p - hi) (p - hi is exact in fp32), so hi + lo is p to about
// 2^-17 relative.  For a 16-token tile the pair fills one 16x16x32 product:
// contraction index 8 g + e holds token 4 g + (e mod 4) of lane group g, with
// hi for e < 4 and lo for e >= 4, and the A operand holds that token's V
// elements twice -- the sum runs over every token's hi and lo term at the
// cost of the single 16x16x16 product that a bf16-rounded P would take.
__device__ __forceinline__ void split_bf16(const float* p, bf16x4& hi, bf16x4& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const __bf16 h = (__bf16)p[i];
    hi[i] = h;
    lo[i] = (__bf16)(p[i] - (float)h);
  }
}
__device__ __forceinline__ bf16x8 twice(bf16x4 v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3, 0, 1, 2, 3); }
__device__ __forceinline__ bf16x8 join(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Online-softmax state of one unit: column col's reference maximum m (base-2
// units, uniform over the four groups) and -m, this lane's share of the
// running sum, and the O^T accumulators.
template <int D>
struct Fold {
  float m, mneg, lsum;
  f32x4 o[Geo<D>::NPV];
  __device__ __forceinline__ void reset() {
    m = -INFINITY;
    mneg = 0.0f;
    lsum = 0.0f;
#pragma unroll
    for (int j = 0; j < Geo<D>::NPV; ++j) o[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
};

// Folds one loaded tile into the unit's state.
template <int D>
__device__ __forceinline__ void fold_tile(uint32_t ok, const u32x4m (&kr)[Geo<D>::NI],
                                          const u32x4m (&vr)[Geo<D>::NI], const bf16x8 (&qop)[Geo<D>::NQK],
                                          float cs, const LdsMap<D>& map, int lane, Fold<D>& st,
                                          uint8_t* __restrict__ lds_k, uint8_t* __restrict__ lds_v) {
  constexpr int PPR = Geo<D>::PPR, NI = Geo<D>::NI, NQK = Geo<D>::NQK, NPV = Geo<D>::NPV;
  const int grp = lane >> 4;
  // Stage the tile in LDS (the previous tile's reads were issued earlier by
  // this wavefront, and LDS serves one wavefront's accesses in order).
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    *reinterpret_cast<u32x4m*>(lds_k + map.wr[u]) = kr[u];
    *reinterpret_cast<u32x4m*>(lds_v + map.wr[u]) = vr[u];
  }
  // S = K_tile . Q^T: lane holds S[token 4 grp + i][head col].
  f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < NQK; ++c) {
    const int pc = 4 * c + grp;
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds_k + (map.tk * PPR + (pc ^ swz<PPR>(map.tk))) * 16);
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
  if (__builtin_amdgcn_ballot_w64(mt > st.m + kSlackM)) {   // wavefront-uniform, rare
    if (mt > st.m) {
      const float corr = exp2m(st.m - mt);                  // 0 while m is -inf
      st.m = mt;
      st.mneg = -mt;
      st.lsum *= corr;
#pragma unroll
      for (int j = 0; j < NPV; ++j) st.o[j] *= corr;
    }
  }
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pr[i] = exp2m(sc[i] + st.mneg);
    st.lsum += pr[i];
  }
  bf16x4 ph, pl;
  split_bf16(pr, ph, pl);
  const bf16x8 pb = join(ph, pl);
  // O^T += V_tile^T . (P_hi + P_lo)^T, one 16-column d chunk per product.
#pragma unroll
  for (int j = 0; j < NPV; ++j) {
    const int d = 16 * j + map.dv;
    const int pc = d >> 3;
    const int addr = (map.tv * PPR + (pc ^ swz<PPR>(map.tv))) * 16 + (d & 7) * 2;
    const s16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(lds_v + addr));
    st.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(twice(__builtin_bit_cast(bf16x4, vt)), pb, st.o[j], 0, 0, 0);
  }
}

// Writes a finished unit: the final bf16 output of a one-partition sequence
// (outside the append step), else the fp32 partial (acc, m, l) of partition p
// for the merge kernel.
template <int D, bool Shared = false>
__device__ __forceinline__ void store_unit(const DecodeParams& prm, const Unit& u, int lane, const Fold<D>& st,
                                           const int32_t* jn) {
  constexpr int NPV = Geo<D>::NPV;
  const int grp = lane >> 4;
  const ColHead c = column_head<Shared>(prm, u, lane & 15, jn);
  const bool head_ok = c.ok;
  const float L = groups_sum(st.lsum);
  const size_t bh = (size_t)c.b * prm.H + c.h;
  // (structured branches only: an early return under the per-lane head_ok
  // would make the compiler treat the caller's later state as divergent)
  if (u.np <= 1 && !prm.append) {
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    uint16_t* outp = static_cast<uint16_t*>(prm.out) + bh * D;
    if (head_ok) {
#pragma unroll
      for (int j = 0; j < NPV; ++j) {
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (__bf16)(st.o[j][i] * inv);
        *reinterpret_cast<bf16x4*>(outp + 16 * j + 4 * grp) = w;
      }
    }
  } else {
    const size_t slot = bh * prm.maxP + u.p;
    float* dst = prm.ws_acc + slot * D;
    if (head_ok) {
#pragma unroll
      for (int j = 0; j < NPV; ++j) *reinterpret_cast<f32x4*>(dst + 16 * j + 4 * grp) = st.o[j];
      if (grp == 0) *reinterpret_cast<float2*>(prm.ws_ml + slot * 2) = make_float2(st.m, L);
    }
  }
}

}  // namespace

// Grid form (sequence counts beyond the persistent form's list): one
// workgroup per unit.  Grid x = (kv head, head chunk) fastest, y = partition,
// z = sequence; units past a sequence's last partition exit at once.
template <int D, bool WholeTile>
__global__ __launch_bounds__(64) void decode_partial_mfma_grid_kernel(const DecodeParams prm) {
  using Gm = Geo<D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[16 * Gm::ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[16 * Gm::ROWB];
  const int lane = threadIdx.x;
  const int b = blockIdx.z, p = blockIdx.y;
  const int kvh = blockIdx.x / prm.nchunks;
  const int n = clamp_len(prm, prm.ctx[b]);
  const Unit u = make_unit(prm, b, p, n, kvh, blockIdx.x - kvh * prm.nchunks);
  if (p >= (u.np > 0 ? u.np : 1)) return;
  // lane l: table entry j_first + l of the partition (0 past its blocks)
  const int j_first = u.t_begin >> prm.bs_log2;
  const int j_end = (u.t_end + prm.bs_mask) >> prm.bs_log2;
  const int tbl = (j_first + lane < j_end) ? prm.tables[(size_t)b * prm.W + j_first + lane] : 0;
  // the partition's first block is also the neighbour's block at that table
  // position: a shared prefix, read with the default cache policy
  const int nbr = neighbour(prm, b);
  const int nbr_blocks = nbr >= 0 ? (clamp_len(prm, prm.ctx[nbr]) + prm.bs_mask) >> prm.bs_log2 : 0;
  const bool shared = j_first < j_end && j_first < nbr_blocks &&
                      prm.tables[(size_t)nbr * prm.W + j_first] == prm.tables[(size_t)b * prm.W + j_first];
  const char* kc = kv_col<D>(prm.k_cache, kvh);
  const char* vc = kv_col<D>(prm.v_cache, kvh);
  u32x4m qr[Gm::NQK];
  load_q<D>(prm, u, lane, qr, nullptr);
  bf16x8 qop[Gm::NQK];
  q_operands<D>(prm, u, lane, qr, qop);
  const LdsMap<D> map(lane);
  const uint32_t lane_off = (uint32_t)(lane / Gm::PPR) * (uint32_t)(prm.KVH * Gm::ROWB) + (uint32_t)(lane % Gm::PPR) * 16;
  Fold<D> st;
  st.reset();
  auto run = [&](auto pol) {
    constexpr int A = decltype(pol)::aux;
    u32x4m kA[Gm::NI], vA[Gm::NI], kB[Gm::NI], vB[Gm::NI];
    auto load_at = [&](int i, u32x4m (&kr)[Gm::NI], u32x4m (&vr)[Gm::NI]) {
      const int tile = u.t_begin + min(i, u.ntiles - 1) * 16;
      const int j = (tile >> prm.bs_log2) - j_first;
      const int ph0 = __builtin_amdgcn_readlane(tbl, j & 63);
      const int ph1 = WholeTile ? ph0 : __builtin_amdgcn_readlane(tbl, (j + 1) & 63);
      return load_tile<D, WholeTile, A>(prm, kc, vc, u.t_end, tile, true, ph0, ph1, lane_off, kr, vr);
    };
    uint32_t okA = load_at(0, kA, vA), okB;
    for (int ip = 0; ip < (u.ntiles >> 1); ++ip) {
      okB = load_at(2 * ip + 1, kB, vB);
      fold_tile<D>(okA, kA, vA, qop, prm.scale_log2, map, lane, st, lds_k, lds_v);
      okA = load_at(2 * ip + 2, kA, vA);
      fold_tile<D>(okB, kB, vB, qop, prm.scale_log2, map, lane, st, lds_k, lds_v);
    }
    if (u.ntiles & 1) fold_tile<D>(okA, kA, vA, qop, prm.scale_log2, map, lane, st, lds_k, lds_v);
  };
  if (shared)
    run(CachePolicy<0>{});
  else
    run(CachePolicy<kAuxNT>{});
  store_unit<D>(prm, u, lane, st, nullptr);
}

// vLLM's cache layout ("PagedAttention kernel：paged KV cache 与 block table",
// 深入原理): K [NB, KVH, D/8, bs, 8], V [NB, KVH, D, bs].  There the operands of
// a 16-token tile load straight from the block in operand order, with no LDS:
//   K (A of S = K Q^T): lane l takes the 16-byte group 4 c + l / 16 of token
//     row l % 16; the 16 lanes of a group read 256 contiguous bytes;
//   V^T (A of O^T += V^T P^T; 16x16x32 with the V elements twice, as for the
//     LDS-staged tiles): lane l takes tokens 4 (l / 16) .. + 3
//     of d row 16 j + l % 16, 8 contiguous bytes.
// Rows past the partition's end, and blocks outside the pool, are not loaded
// (zeros); V elements of rows past the end are zeroed, so stale values never
// reach the products.
namespace {

typedef uint32_t u32x2m __attribute__((ext_vector_type(2)));

template <int D>
struct VllmTile {
  u32x4m k[Geo<D>::NQK];
  u32x2m v[Geo<D>::NPV];
};

// Loads the 16-token tile starting at token `tile` (block ph0; for block size
// 8 the tile's second half is block ph1) of kv head kvh, valid rows
// [0, t_end - tile).  Buffer loads, one resource per block over the kv head's
// region of it (empty for a block outside the pool), so that nothing branches
// around a load; a lane whose row lies in the other block of a split tile
// reads past its resource's end (zeros).  V elements of rows past the end are
// zeroed.  Returns the row validity mask.
template <int D, bool WholeTile, int AUX = 0>
__device__ __forceinline__ uint32_t load_tile_vllm(const DecodeParams& prm, int kvh, int t_end, int tile,
                                                   int ph0, int ph1, int lane, VllmTile<D>& T) {
  constexpr int NQK = Geo<D>::NQK, NPV = Geo<D>::NPV;
  constexpr uint32_t kFar = 0x80000000u;   // a byte offset past every resource's end
  const int bs_log2 = prm.bs_log2;
  const int nv = min(16, t_end - tile);
  const int r = lane & 15, g4 = lane >> 4;
  const bool ok0 = (unsigned)ph0 < (unsigned)prm.NB, ok1 = (unsigned)ph1 < (unsigned)prm.NB;
  const int k_region = (D / 8) << (bs_log2 + 4), v_region = D << (bs_log2 + 1);   // bytes per (block, kv head)
  auto rsrc = [&](const void* cache, int blk, bool ok, int region) {
    const char* base = static_cast<const char*>(cache) + (size_t)(ok ? blk : 0) * prm.KVH * region + (size_t)kvh * region;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, ok ? region : 0, kRsrcWord3M);
  };
  const int row0 = WholeTile ? (tile & prm.bs_mask) : 0;
  // K: token row r of the tile
  {
    const int krow = WholeTile ? row0 + r : (r & 7);
    const __amdgpu_buffer_rsrc_t k0 = rsrc(prm.k_cache, ph0, ok0, k_region);
#pragma unroll
    for (int c = 0; c < NQK; ++c) {
      const uint32_t off = ((uint32_t)((4 * c + g4) << bs_log2) + krow) * 16;
      if constexpr (WholeTile) {
        T.k[c] = __builtin_amdgcn_raw_buffer_load_b128(k0, off, 0, AUX);
      } else {
        const __amdgpu_buffer_rsrc_t k1 = rsrc(prm.k_cache, ph1, ok1, k_region);
        const u32x4m a = __builtin_amdgcn_raw_buffer_load_b128(k0, r < 8 ? off : kFar, 0, AUX);
        const u32x4m b = __builtin_amdgcn_raw_buffer_load_b128(k1, r < 8 ? kFar : off, 0, AUX);
        T.k[c] = a | b;
      }
    }
  }
  // V: tokens 4 g4 .. 4 g4 + 3 of d rows 16 j + r
  {
    const int vtok = WholeTile ? row0 + 4 * g4 : ((4 * g4) & 7);
    const int vn = min(max(nv - 4 * g4, 0), 4);            // valid tokens of the lane's 4
    const uint32_t keep_lo = vn >= 2 ? 0xffffffffu : (vn == 1 ? 0x0000ffffu : 0u);
    const uint32_t keep_hi = vn >= 4 ? 0xffffffffu : (vn == 3 ? 0x0000ffffu : 0u);
    const __amdgpu_buffer_rsrc_t v0 = rsrc(prm.v_cache, ph0, ok0, v_region);
#pragma unroll
    for (int j = 0; j < NPV; ++j) {
      const uint32_t off = ((uint32_t)((16 * j + r) << bs_log2) + vtok) * 2;
      u32x2m w;
      if constexpr (WholeTile) {
        w = __builtin_amdgcn_raw_buffer_load_b64(v0, off, 0, AUX);
      } else {
        const __amdgpu_buffer_rsrc_t v1 = rsrc(prm.v_cache, ph1, ok1, v_region);
        const u32x2m a = __builtin_amdgcn_raw_buffer_load_b64(v0, g4 < 2 ? off : kFar, 0, AUX);
        const u32x2m b = __builtin_amdgcn_raw_buffer_load_b64(v1, g4 < 2 ? kFar : off, 0, AUX);
        w = a | b;
      }
      w[0] &= keep_lo;
      w[1] &= keep_hi;
      T.v[j] = w;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  uint32_t ok;
  if constexpr (WholeTile) {
    ok = ok0 ? (nv >= 16 ? 0xffffu : (nv > 0 ? (1u << nv) - 1u : 0u)) : 0u;
  } else {
    const uint32_t lo = ok0 ? (nv >= 8 ? 0xffu : (nv > 0 ? (1u << nv) - 1u : 0u)) : 0u;
    const uint32_t hi = ok1 && nv > 8 ? ((nv >= 16 ? 0xffu : (1u << (nv - 8)) - 1u) << 8) : 0u;
    ok = lo | hi;
  }
  return ok;
}

// Folds a tile held in registers: S = K . Q^T, the same online softmax as the
// LDS-staged tiles (scores masked by row validity, lazy rescale, P^T as a
// hi + lo pair of bf16), and O^T += V^T . P^T.
template <int D>
__device__ __forceinline__ void fold_tile_vllm(uint32_t ok, const VllmTile<D>& T, const bf16x8 (&qop)[Geo<D>::NQK],
                                               float cs, int lane, Fold<D>& st) {
  constexpr int NQK = Geo<D>::NQK, NPV = Geo<D>::NPV;
  const int grp = lane >> 4;
  f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < NQK; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, T.k[c]), qop[c], s, 0, 0, 0);
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] = ((ok >> (4 * grp + i)) & 1u) ? s[i] * cs : -INFINITY;
  float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  mt = groups_max(mt);
  if (__builtin_amdgcn_ballot_w64(mt > st.m + kSlackM)) {
    if (mt > st.m) {
      const float corr = exp2m(st.m - mt);
      st.m = mt;
      st.mneg = -mt;
      st.lsum *= corr;
#pragma unroll
      for (int j = 0; j < NPV; ++j) st.o[j] *= corr;
    }
  }
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pr[i] = exp2m(sc[i] + st.mneg);
    st.lsum += pr[i];
  }
  bf16x4 ph, pl;
  split_bf16(pr, ph, pl);
  const bf16x8 pb = join(ph, pl);
#pragma unroll
  for (int j = 0; j < NPV; ++j)
    st.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(twice(__builtin_bit_cast(bf16x4, T.v[j])), pb, st.o[j], 0, 0,
                                                      0);
}

// 32-token tiles for blocks of 32 tokens or more (a tile then lies in one
// block): a 16-token tile reads half of every K group and V row of such a
// block, a 32-token one reads whole K groups (512 bytes for 32 tokens) and
// whole 64-byte V rows.
//   K: k[h][c] is the 16-byte group 4 c + l / 16 of token row 16 h + l % 16.
//   V^T as the A operand of v_mfma_f32_16x16x32_bf16 (d rows x 32 keys): lane
//     l holds d row 16 j + l % 16 at contraction indices 8 (l / 16) + e, taken
//     to be keys 4 (l / 16) + e (e < 4) and 16 + 4 (l / 16) + e - 4 (e >= 4):
//     two 8-byte reads of the row.  The probabilities use the same order:
//     S accumulator h of lane l holds keys 16 h + 4 (l / 16) + i, so the B
//     operand is (P of accumulator 0, P of accumulator 1) with no data
//     movement, and the product sums over all 32 keys.
template <int D>
struct VllmTile32 {
  u32x4m k[2][Geo<D>::NQK];
  u32x4m v[Geo<D>::NPV];
};

template <int D, int AUX = 0>
__device__ __forceinline__ uint32_t load_tile_vllm32(const DecodeParams& prm, int kvh, int t_end, int tile,
                                                     int ph0, int lane, VllmTile32<D>& T) {
  constexpr int NQK = Geo<D>::NQK, NPV = Geo<D>::NPV;
  const int bs_log2 = prm.bs_log2;
  const int nv = min(32, t_end - tile);
  const int r = lane & 15, g4 = lane >> 4;
  const bool ok0 = (unsigned)ph0 < (unsigned)prm.NB;
  const int k_region = (D / 8) << (bs_log2 + 4), v_region = D << (bs_log2 + 1);   // bytes per (block, kv head)
  auto rsrc = [&](const void* cache, int region) {
    const char* base = static_cast<const char*>(cache) + (size_t)(ok0 ? ph0 : 0) * prm.KVH * region + (size_t)kvh * region;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, ok0 ? region : 0, kRsrcWord3M);
  };
  const int row0 = tile & prm.bs_mask;
  const __amdgpu_buffer_rsrc_t k0 = rsrc(prm.k_cache, k_region);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int c = 0; c < NQK; ++c) {
      const uint32_t off = ((uint32_t)((4 * c + g4) << bs_log2) + row0 + 16 * h + r) * 16;
      T.k[h][c] = __builtin_amdgcn_raw_buffer_load_b128(k0, off, 0, AUX);
    }
  const int vlo = min(max(nv - 4 * g4, 0), 4), vhi = min(max(nv - 16 - 4 * g4, 0), 4);   // valid tokens
  auto keep = [](int vn, int half) {          // mask of the 32-bit word `half` of 4 tokens, vn valid
    const int k = vn - 2 * half;
    return k >= 2 ? 0xffffffffu : (k == 1 ? 0x0000ffffu : 0u);
  };
  const uint32_t m0 = keep(vlo, 0), m1 = keep(vlo, 1), m2 = keep(vhi, 0), m3 = keep(vhi, 1);
  const __amdgpu_buffer_rsrc_t v0 = rsrc(prm.v_cache, v_region);
#pragma unroll
  for (int j = 0; j < NPV; ++j) {
    const uint32_t off = ((uint32_t)((16 * j + r) << bs_log2) + row0 + 4 * g4) * 2;
    const u32x2m lo = __builtin_amdgcn_raw_buffer_load_b64(v0, off, 0, AUX);
    const u32x2m hi = __builtin_amdgcn_raw_buffer_load_b64(v0, off + 32, 0, AUX);
    T.v[j] = u32x4m{lo[0] & m0, lo[1] & m1, hi[0] & m2, hi[1] & m3};
  }
  __builtin_amdgcn_sched_barrier(0);
  return ok0 && nv > 0 ? (nv >= 32 ? 0xffffffffu : (1u << nv) - 1u) : 0u;
}

template <int D>
__device__ __forceinline__ void fold_tile_vllm32(uint32_t ok, const VllmTile32<D>& T,
                                                 const bf16x8 (&qop)[Geo<D>::NQK], float cs, int lane, Fold<D>& st) {
  constexpr int NQK = Geo<D>::NQK, NPV = Geo<D>::NPV;
  const int grp = lane >> 4;
  f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < NQK; ++c) {
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, T.k[0][c]), qop[c], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, T.k[1][c]), qop[c], s1, 0, 0, 0);
  }
  float sc[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[i] = ((ok >> (4 * grp + i)) & 1u) ? s0[i] * cs : -INFINITY;
    sc[4 + i] = ((ok >> (16 + 4 * grp + i)) & 1u) ? s1[i] * cs : -INFINITY;
  }
  float mt = sc[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sc[i]);
  mt = groups_max(mt);
  if (__builtin_amdgcn_ballot_w64(mt > st.m + kSlackM)) {
    if (mt > st.m) {
      const float corr = exp2m(st.m - mt);
      st.m = mt;
      st.mneg = -mt;
      st.lsum *= corr;
#pragma unroll
      for (int j = 0; j < NPV; ++j) st.o[j] *= corr;
    }
  }
  float pr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pr[i] = exp2m(sc[i] + st.mneg);
    st.lsum += pr[i];
  }
  // P = hi + lo as two products over the tile's 32 keys
  bf16x4 h0, l0, h1, l1;
  split_bf16(pr, h0, l0);
  split_bf16(pr + 4, h1, l1);
  const bf16x8 phi = join(h0, h1), plo = join(l0, l1);
#pragma unroll
  for (int j = 0; j < NPV; ++j) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, T.v[j]);
    st.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, phi, st.o[j], 0, 0, 0);
    st.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, plo, st.o[j], 0, 0, 0);
  }
}

}  // namespace

// One wavefront per unit (kv head and head chunk fastest, partition,
// sequence), tiles double-buffered in registers.
template <int D, bool WholeTile>
__global__ __launch_bounds__(64) void decode_partial_vllm_kernel(const DecodeParams prm) {
  const int lane = threadIdx.x;
  const int b = blockIdx.z, p = blockIdx.y;
  const int kvh = blockIdx.x / prm.nchunks;
  const int n = clamp_len(prm, prm.ctx[b]);
  const Unit u = make_unit(prm, b, p, n, kvh, blockIdx.x - kvh * prm.nchunks);
  if (p >= (u.np > 0 ? u.np : 1)) return;
  const int j_first = u.t_begin >> prm.bs_log2;
  const int j_end = (u.t_end + prm.bs_mask) >> prm.bs_log2;
  const int tbl = (j_first + lane < j_end) ? prm.tables[(size_t)b * prm.W + j_first + lane] : -1;
  u32x4m qr[Geo<D>::NQK];
  load_q<D>(prm, u, lane, qr, nullptr);
  bf16x8 qop[Geo<D>::NQK];
  q_operands<D>(prm, u, lane, qr, qop);
  Fold<D> st;
  st.reset();
  VllmTile<D> A, Bt;
  auto load_at = [&](int i, VllmTile<D>& T) {
    const int tile = u.t_begin + min(i, u.ntiles - 1) * 16;
    const int j = (tile >> prm.bs_log2) - j_first;
    const int ph0 = __builtin_amdgcn_readlane(tbl, j & 63);
    const int ph1 = WholeTile ? ph0 : __builtin_amdgcn_readlane(tbl, (j + 1) & 63);
    return load_tile_vllm<D, WholeTile>(prm, kvh, u.t_end, tile, ph0, ph1, lane, T);
  };
  uint32_t okA = load_at(0, A), okB;
  for (int ip = 0; ip < (u.ntiles >> 1); ++ip) {
    okB = load_at(2 * ip + 1, Bt);
    fold_tile_vllm<D>(okA, A, qop, prm.scale_log2, lane, st);
    okA = load_at(2 * ip + 2, A);
    fold_tile_vllm<D>(okB, Bt, qop, prm.scale_log2, lane, st);
  }
  if (u.ntiles & 1) fold_tile_vllm<D>(okA, A, qop, prm.scale_log2, lane, st);
  store_unit<D>(prm, u, lane, st, nullptr);
}

namespace {

// What the persistent walk needs from a cache layout: a tile's registers, its
// load and its fold.
template <int D>
struct P09Tile {
  u32x4m k[Geo<D>::NI], v[Geo<D>::NI];
};

template <int D, bool WholeTile, bool Vllm, int TOK = 16>
struct TileOps;

template <int D, bool WholeTile>
struct TileOps<D, WholeTile, false, 16> {   // P09 layout: whole rows, staged through LDS
  using Tile = P09Tile<D>;
  template <int AUX>
  static __device__ __forceinline__ uint32_t load(const DecodeParams& prm, int kvh, int t_end, int tile, bool live,
                                                  int ph0, int ph1, int lane, uint32_t lane_off, Tile& T) {
    return load_tile<D, WholeTile, AUX>(prm, kv_col<D>(prm.k_cache, kvh), kv_col<D>(prm.v_cache, kvh), t_end,
                                        tile, live, ph0, ph1, lane_off, T.k, T.v);
  }
  static __device__ __forceinline__ void fold(uint32_t ok, const Tile& T, const bf16x8 (&qop)[Geo<D>::NQK],
                                              float cs, const LdsMap<D>& map, int lane, Fold<D>& st,
                                              uint8_t* lds_k, uint8_t* lds_v) {
    fold_tile<D>(ok, T.k, T.v, qop, cs, map, lane, st, lds_k, lds_v);
  }
};

template <int D, bool WholeTile>
struct TileOps<D, WholeTile, true, 16> {    // vLLM layout: operands straight from the blocks
  using Tile = VllmTile<D>;
  template <int AUX>
  static __device__ __forceinline__ uint32_t load(const DecodeParams& prm, int kvh, int t_end, int tile, bool live,
                                                  int ph0, int ph1, int lane, uint32_t, Tile& T) {
    return load_tile_vllm<D, WholeTile, AUX>(prm, kvh, t_end, tile, live ? ph0 : -1, live ? ph1 : -1, lane, T);
  }
  static __device__ __forceinline__ void fold(uint32_t ok, const Tile& T, const bf16x8 (&qop)[Geo<D>::NQK],
                                              float cs, const LdsMap<D>&, int lane, Fold<D>& st, uint8_t*,
                                              uint8_t*) {
    fold_tile_vllm<D>(ok, T, qop, cs, lane, st);
  }
};

template <int D>
struct TileOps<D, true, true, 32> {     // vLLM layout, blocks of 32 tokens or more: 32-token tiles
  using Tile = VllmTile32<D>;
  template <int AUX>
  static __device__ __forceinline__ uint32_t load(const DecodeParams& prm, int kvh, int t_end, int tile, bool live,
                                                  int ph0, int, int lane, uint32_t, Tile& T) {
    return load_tile_vllm32<D, AUX>(prm, kvh, t_end, tile, live ? ph0 : -1, lane, T);
  }
  static __device__ __forceinline__ void fold(uint32_t ok, const Tile& T, const bf16x8 (&qop)[Geo<D>::NQK],
                                              float cs, const LdsMap<D>&, int lane, Fold<D>& st, uint8_t*,
                                              uint8_t*) {
    fold_tile_vllm32<D>(ok, T, qop, cs, lane, st);
  }
};

}  // namespace

// Persistent form: one workgroup of NW wavefronts per CU; each wavefront folds
// a sequence of units as one continuous stream of tiles: the loads of a
// unit's first tile (and its q) are issued while the previous unit's last
// tile is folded, so no unit starts with an empty pipeline.
//
// The unit list (built in LDS by the workgroup's first wavefront from the
// context lengths, so that all workgroups agree on it without
// communication): first every sequence's partitions before its last one (all
// full, P tokens), sequence by sequence, then the last partition of each
// sequence in decreasing length (counting sort over kBuckets length
// classes), so that the shortest units come last; each (sequence, partition)
// pair expands into kv heads x head chunks consecutive units.
//
// Workgroup c of NC owns one unit of every round of NC units (round k dealt
// in serpentine order, below).  Inside the workgroup the units are handed out in that
// order through an LDS counter as wavefronts finish their previous one:
// wavefronts sharing a CU stream at very different rates, and this lets the
// faster ones take more units, so that all of a CU's wavefronts finish
// together.
template <int D, bool WholeTile, int NW, bool Vllm = false, int TOK = 16>
__global__ __launch_bounds__(64 * NW) void decode_partial_mfma_kernel(const DecodeParams prm) {
  using Gm = Geo<D>;
  using Ops = TileOps<D, WholeTile, Vllm, TOK>;
  using Tile = typename Ops::Tile;
  constexpr int NBUF = 2;   // tiles in flight per wavefront (3 measured no faster)
  __shared__ __attribute__((aligned(16))) uint8_t lds_tiles[NW][2][16 * Gm::ROWB];
  __shared__ int32_t s_cnt[kBuckets];
  __shared__ uint32_t s_next;         // next unit (in the workgroup's share) to hand out
  __shared__ int32_t s_shared;        // some sequence starts with its neighbour's first block
  __shared__ int32_t s_nj;            // sequences that fold the shared partitions in shared units
  extern __shared__ int32_t s_list[];
  const int B = prm.B, P = prm.P;
  int32_t* s_first = s_list;          // [B] list index of sequence b's first full pair
  int32_t* s_len = s_list + B;        // [B] clamped context length
  int32_t* s_last = s_list + 2 * B;   // [B] sequences in last-pair order
  int32_t* s_skip = s_list + 3 * B;   // [B] leading partitions sequence b leaves to shared units (0 or SP)
  int32_t* s_jn = s_list + 4 * B;     // [s_nj] those sequences, in order
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t NC = gridDim.x, wg = blockIdx.x;
#ifdef PA_TIMELINE
  const uint64_t tl_entry = __builtin_amdgcn_s_memrealtime();
#endif
  uint8_t* lds_k = lds_tiles[wave][0];
  uint8_t* lds_v = lds_tiles[wave][1];

  // ---- the unit list (first wavefront) ----
  const int tmax = (P + 15) >> 4;     // tiles of a full partition
  auto last_class = [&](int n) {      // 0 = longest last partition
    const int np = (n + P - 1) / P;
    const int lt = (n - (np > 1 ? (np - 1) * P : 0) + 15) >> 4;
    return (kBuckets - 1) - lt * (kBuckets - 1) / tmax;
  };
  // Shared prefix: every wavefront compares a share of the (sequence, entry)
  // pairs of the shared partitions with row 0 (SP * P <= W * bs keeps every
  // entry inside its row); a mismatch marks the sequence in s_skip (all
  // writers store 1).  Loads go out 16 at a time at clamped indices.  When
  // the rows are 16-byte aligned (the table 16-byte aligned, W a multiple of
  // 4) a load compares 4 entries: the quads cover entries up to
  // 4 * ceil(SPB / 4) <= W, and entries past SPB are ignored.  When a row's
  // quads fit in the workgroup, thread t keeps quad column j = t mod spb4 for
  // rows t / spb4 + k * rpp (row 0's quad is loaded once), and its first 16
  // rows' loads go out before the length copy below, so that both wait for
  // memory together (the first pass is compared into a register mask, and
  // marked after the barrier that orders the marks after the zeroing).
  //
  // Every wavefront also copies each sequence's clamped length and its first
  // table entry (every row has one) into LDS, so that the list wavefront reads
  // them from LDS: one round trip to memory instead of one per 64 sequences.
  // s_last holds the entries until the list wavefront overwrites it with the
  // last-pair order, after its last use of them.
  const int b_first = (int)threadIdx.x;
  int len_first = 0, ent_first = 0;
  if (b_first < B) {
    len_first = prm.ctx[b_first];
    ent_first = prm.tables[(size_t)b_first * prm.W];
  }
  typedef int32_t i32x4t __attribute__((ext_vector_type(4)));
  constexpr int kU = 16;
  const int spb = prm.SPB;
  const bool quads = prm.SP > 0 && (prm.W & 3) == 0 && (reinterpret_cast<uintptr_t>(prm.tables) & 15u) == 0;
  const i32x4t* t4 = reinterpret_cast<const i32x4t*>(prm.tables);
  const int spb4 = (spb + 3) >> 2, w4 = prm.W >> 2;
  const int rpp = quads ? (64 * NW) / spb4 : 0;       // rows per pass of the workgroup
  const bool fixed_col = rpp > 0 && (int)threadIdx.x < rpp * spb4;
  const int jcol = fixed_col ? (int)threadIdx.x % spb4 : 0;
  const int brow = fixed_col ? (int)threadIdx.x / spb4 : 0;
  i32x4t ref4 = {0, 0, 0, 0}, mine4[kU];
  auto differs = [&](const i32x4t& m) {
    bool diff = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) diff |= (4 * jcol + i < spb) && m[i] != ref4[i];
    return diff;
  };
  uint32_t miss = 0;   // bit u: row brow + u * rpp of the first pass differs from row 0
  if (fixed_col) {
    ref4 = t4[jcol];
#pragma unroll
    for (int u = 0; u < kU; ++u) mine4[u] = t4[(size_t)min(brow + u * rpp, B - 1) * w4 + jcol];
#pragma unroll
    for (int u = 0; u < kU; ++u) miss |= differs(mine4[u]) ? 1u << u : 0u;
  }
  if (b_first < B) {
    s_len[b_first] = clamp_len(prm, len_first);
    s_last[b_first] = ent_first;
    s_skip[b_first] = 0;
  }
  for (int b = b_first + 64 * NW; b < B; b += 64 * NW) {
    s_len[b] = clamp_len(prm, prm.ctx[b]);
    s_last[b] = prm.tables[(size_t)b * prm.W];
    s_skip[b] = 0;
  }
  __syncthreads();
  if (prm.SP > 0) {
    if (fixed_col) {
      for (int b0 = brow;; b0 += rpp * kU) {
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (((miss >> u) & 1u) && b0 + u * rpp < B) s_skip[b0 + u * rpp] = 1;
        if (b0 + rpp * kU >= B) break;
#pragma unroll
        for (int u = 0; u < kU; ++u) mine4[u] = t4[(size_t)min(b0 + rpp * kU + u * rpp, B - 1) * w4 + jcol];
        miss = 0;
#pragma unroll
        for (int u = 0; u < kU; ++u) miss |= differs(mine4[u]) ? 1u << u : 0u;
      }
    }
    if (quads && rpp == 0) {
      const int total4 = B * spb4;
      for (int e0 = threadIdx.x; e0 < total4; e0 += 64 * NW * kU) {
        i32x4t mine[kU], ref[kU];
        int who[kU], jq[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int e = min(e0 + u * 64 * NW, total4 - 1);
          const int b = e / spb4, j = e - b * spb4;
          who[u] = b;
          jq[u] = j;
          mine[u] = t4[(size_t)b * w4 + j];
          ref[u] = t4[j];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          bool diff = false;
#pragma unroll
          for (int i = 0; i < 4; ++i) diff |= (4 * jq[u] + i < spb) && mine[u][i] != ref[u][i];
          if (diff) s_skip[who[u]] = 1;
        }
      }
    }
    const int total = quads ? 0 : B * spb;   // rows not 16-byte aligned: one entry per load
    for (int e0 = threadIdx.x; e0 < total; e0 += 64 * NW * kU) {
      int mine[kU], ref[kU], who[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int e = min(e0 + u * 64 * NW, total - 1);
        const int b = e / spb, j = e - b * spb;
        who[u] = b;
        mine[u] = prm.tables[(size_t)b * prm.W + j];
        ref[u] = prm.tables[j];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (mine[u] != ref[u]) s_skip[who[u]] = 1;
    }
    __syncthreads();
  }
  if (wave == 0) {
    s_cnt[lane] = 0;
    if (lane == 0) s_next = NW;
    int carry = 0, jcarry = 0;
    bool shared = false;
    for (int base = 0; base < B; base += 64) {
      const int b = base + lane;
      const int n = b < B ? s_len[b] : 0;
      {
        // entry 0 of every table row exists; it is compared only when both
        // sequences use it
        const int nb = b < B ? neighbour(prm, b) : -1;
        const int nn = nb >= 0 ? s_len[nb] : 0;
        const int e0 = b < B ? s_last[b] : -1;
        const int e1 = nb >= 0 ? s_last[nb] : -2;
        shared |= __ballot(n > 0 && nn > 0 && e0 == e1) != 0;
      }
      // Shared prefix: the sequence leaves its first SP partitions to shared
      // units when its context extends past them and its first SPB table
      // entries equal row 0's (no mismatch marked above).
      const bool join = prm.SP > 0 && b < B && n > prm.SP * P && s_skip[b] == 0;
      const uint64_t jm = __ballot(join);
      if (join) s_jn[jcarry + __popcll(jm & ((1ull << lane) - 1ull))] = b;
      jcarry += __popcll(jm);
      shared |= jm != 0;
      const int np = (n + P - 1) / P;
      const int f = (b < B && np > 1) ? np - 1 - (join ? prm.SP : 0) : 0;
      const int incl = wave_inclusive_sum(f);
      if (b < B) {
        s_first[b] = carry + incl - f;
        s_skip[b] = join ? prm.SP : 0;
        atomicAdd(&s_cnt[last_class(n)], 1);
      }
      carry += __builtin_amdgcn_readlane(incl, 63);
    }
    {
      const int c = s_cnt[lane];
      s_cnt[lane] = wave_inclusive_sum(c) - c;
    }
    for (int base = 0; base < B; base += 64) {
      const int b = base + lane;
      if (b < B) s_last[atomicAdd(&s_cnt[last_class(s_len[b])], 1)] = b;
    }
    if (lane == 0) {
      s_shared = shared ? 1 : 0;
      s_cnt[0] = carry;               // pairs of full partitions (the bucket bases are no longer needed)
      s_nj = jcarry;
    }
  }
  __syncthreads();

#ifdef PA_TIMELINE
  const uint64_t tl_list = __builtin_amdgcn_s_memrealtime();
#endif
  const uint32_t F = (uint32_t)__builtin_amdgcn_readfirstlane(s_cnt[0]);   // pairs of full partitions
  const int nj = __builtin_amdgcn_readfirstlane(s_nj);
  const int SG = prm.SG > 0 ? prm.SG : 1;
  // shared pairs (shared partition, group of SG sequences), listed first: they
  // are full partitions
  const uint32_t NG = prm.SP > 0 ? (uint32_t)((nj + SG - 1) / SG) : 0u;
  const uint32_t SPG = (uint32_t)prm.SP * NG;
  const uint32_t upp = (uint32_t)(prm.KVH * prm.nchunks);
  const uint32_t nunits = (SPG + F + (uint32_t)B) * upp;
  const int stride = (B + 63) >> 6;                   // sequences per lane in the first search level

  // (one return path: units built on several paths end up in scratch memory)
  // The workgroup's k-th unit: round k of the list, dealt to the workgroups in
  // order when k is even and in reverse order when k is odd (a serpentine
  // deal: the list runs from the largest units to the smallest, so a
  // workgroup that drew a larger unit in one round draws a smaller one in the
  // next).  Dealing every round in the same order left up to one extra large
  // unit on some CUs whenever a size class did not fill whole rounds.  Each
  // round is a bijection onto its NC units, and once a workgroup's share lies
  // past the list every later share does too.
  auto share = [&](uint32_t k) { return k * NC + ((k & 1u) ? NC - 1u - wg : wg); };

  auto describe = [&](uint32_t t) -> Unit {
    uint32_t pair = t / upp;
    const uint32_t sub = t - pair * upp;
    int b, p, n, ns = 0, g0 = 0;
    if (pair < SPG) {
      // shared partition sp for group g: a unit over [sp P, (sp + 1) P) whose
      // members all have further partitions (n = (SP + 1) P stands for them)
      const uint32_t sp = pair / NG, g = pair - sp * NG;
      g0 = (int)g * SG;
      ns = min(SG, nj - g0);
      b = __builtin_amdgcn_readfirstlane(s_jn[g0]);
      p = (int)sp;
      n = (prm.SP + 1) * P;
    } else {
      pair -= SPG;
      if (pair < F) {
        // b = the last sequence whose first list index is <= pair: one ballot
        // over every stride-th sequence, then one inside the chosen stretch
        const int i1 = lane * stride;
        const uint64_t m1 = __ballot(i1 < B && (uint32_t)s_first[i1 < B ? i1 : 0] <= pair);
        const int seg = __popcll(m1) - 1;
        const int i2 = seg * stride + lane;
        const uint64_t m2 = __ballot(lane < stride && i2 < B && (uint32_t)s_first[i2 < B ? i2 : 0] <= pair);
        b = __builtin_amdgcn_readfirstlane(seg * stride + __popcll(m2) - 1);
        p = (int)(pair - (uint32_t)__builtin_amdgcn_readfirstlane(s_first[b])) +
            __builtin_amdgcn_readfirstlane(s_skip[b]);
      } else {
        b = __builtin_amdgcn_readfirstlane(s_last[pair - F]);
        p = -1;
      }
      n = __builtin_amdgcn_readfirstlane(s_len[b]);
      if (p < 0) {
        const int np = (n + P - 1) / P;
        p = np > 0 ? np - 1 : 0;
      }
    }
    const int kvh = (int)(sub / (uint32_t)prm.nchunks);
    Unit u = make_unit<TOK>(prm, b, p, n, kvh, (int)sub - kvh * prm.nchunks);
    u.ns = ns;
    u.g0 = g0;
    return u;
  };

  // Folds units from list index t_first on, drawing further ones from the
  // workgroup's queue while they lie below t_stop; returns the first unit
  // drawn at or past t_stop (a later walk starts there).
  auto walk = [&](auto pol, uint32_t t_first, uint32_t t_stop) -> uint32_t {
    constexpr int A = decltype(pol)::aux;
    const LdsMap<D> map(lane);
    const uint32_t lane_off = (uint32_t)(lane / Gm::PPR) * (uint32_t)(prm.KVH * Gm::ROWB) + (uint32_t)(lane % Gm::PPR) * 16;
    const float cs = prm.scale_log2;
    // Block-table entries are read with scalar loads (uniform addresses), one
    // tile ahead of the buffer loads that use them.
    typedef const __attribute__((address_space(4))) int32_t ctab_t;
    ctab_t* ctab = (ctab_t*)prm.tables;

    // State flags of the walk, kept in one word (separate bool variables
    // updated on different paths get merged by the compiler into stores
    // through a selected address, which keeps them in scratch memory):
    //   kNOk     N exists
    //   kNTaken  the producer has moved on to N
    //   kDead    the producer has no further unit
    //   kPending the producer waits for the unit after N
    //   kAlive   the walk goes on
    enum : uint32_t { kNOk = 1, kNTaken = 2, kDead = 4, kPending = 8, kAlive = 16 };
    uint32_t fl = kAlive;
    auto has = [&](uint32_t f) { return (fl & f) != 0; };

    // C: the unit being folded; N: the next one.
    Unit C = describe(t_first);
    Unit N = C;
    uint32_t carry = nunits;
    auto next_unit = [&]() {
      uint32_t k = 0;
      if (lane == 0) k = atomicAdd(&s_next, 1u);
      k = __builtin_amdgcn_readlane(k, 0);
      const uint32_t un = share(k);
      fl = un < t_stop ? (fl | kNOk) : (fl & ~kNOk);
      carry = un < t_stop ? carry : un;
      if (un < t_stop) N = describe(un);
    };
    next_unit();

    u32x4m qr[Gm::NQK], qn[Gm::NQK];
    load_q<D, true>(prm, C, lane, qr, s_jn);
    bf16x8 qop[Gm::NQK];
    q_operands<D>(prm, C, lane, qr, qop);
    Fold<D> st;
    st.reset();
    int c_tile = 0;            // tiles of C folded
#ifdef PA_TIMELINE
    uint64_t tl_unit = __builtin_amdgcn_s_memrealtime();
#endif
    // Producer cursor: the next tile to load is tile l_tile of unit L (C, or
    // N once taken, whose q then goes to qn), with block ids ph0/ph1
    // requested by scalar loads when the cursor moved there (dead: there is
    // no further unit).
    Unit L = C;
    int l_tile = 0, ph0 = -1, ph1 = -1;

    auto request_blocks = [&]() {
      const int tile = L.t_begin + TOK * l_tile;
      const int j = tile >> prm.bs_log2;
      ph0 = -1;
      ph1 = -1;
      if (tile < L.t_end) ph0 = ctab[(size_t)L.b * prm.W + j];
      if (!WholeTile && tile + 8 < L.t_end) ph1 = ctab[(size_t)L.b * prm.W + j + 1];
    };
    // Loads the next tile of the stream into (kr, vr); returns whether it is
    // a real tile (false: the stream is dead, or waits for a unit the
    // consumer has not handed out yet).
    auto produce = [&](Tile& T, uint32_t& ok) -> bool {
      // L exhausted: move on to N (its q first, so that it is older than the
      // tile loads the fold of N's first tile waits for), or wait for the
      // consumer to hand N out, or stop.  (Flags are assigned outright: a
      // store chosen between two flags would keep them in scratch memory.)
      const bool exhausted = !has(kDead | kPending) && l_tile >= L.ntiles;
      if (exhausted) fl |= !has(kNOk) ? kDead : (has(kNTaken) ? kPending : kNTaken);
      if (exhausted && has(kNOk) && (fl & kPending) == 0) {
        L = N;
        l_tile = 0;
        load_q<D, true>(prm, N, lane, qn, s_jn);
        request_blocks();
      }
      const bool live = (fl & (kDead | kPending | kAlive)) == kAlive;
      ok = Ops::template load<A>(prm, L.kvh, L.t_end, L.t_begin + TOK * l_tile, live, ph0, ph1, lane, lane_off, T);
      if (live) {
        ++l_tile;
        if (l_tile < L.ntiles) request_blocks();
      }
      return live;
    };
    // Folds one tile of C; at C's last tile, writes C and moves to N, or
    // ends the walk (alive = false) when there is no further unit.
    auto consume = [&](bool real, uint32_t ok, const Tile& T) {
      if (!real || !has(kAlive)) return;
      Ops::fold(ok, T, qop, cs, map, lane, st, lds_k, lds_v);
      if (++c_tile < C.ntiles) return;
      store_unit<D, true>(prm, C, lane, st, s_jn);
#ifdef PA_TIMELINE
      {
        const uint64_t now = __builtin_amdgcn_s_memrealtime();
        if (lane == 0) {
          const uint32_t u = atomicAdd(reinterpret_cast<unsigned int*>(&g_timeline[0]), 1u);
          if (u < (uint32_t)kTlMaxUnits) {
            uint64_t* r = g_timeline + kTlUnitBase + (size_t)u * 4;
            r[0] = ((uint64_t)wg << 8) | (uint64_t)wave;
            r[1] = ((uint64_t)C.b << 40) | ((uint64_t)C.p << 24) | ((uint64_t)C.kvh << 16) | (uint64_t)C.ntiles;
            r[2] = tl_unit;
            r[3] = now;
          }
        }
        tl_unit = now;
      }
#endif
      if (!has(kNOk)) {
        fl &= ~kAlive;
        return;
      }
      // the tiles of a unit are loaded after all of the previous unit's, so
      // the producer has taken N by now
      C = N;
      q_operands<D>(prm, C, lane, qn, qop);
      st.reset();
      c_tile = 0;
      fl &= ~(kNTaken | kPending);   // a waiting producer moves on at its next load
      next_unit();
    };

    // NBUF tiles in flight: the producer runs NBUF-1 tiles ahead of the
    // folds, in a rotation of register buffers.
    request_blocks();
    Tile tA, tB;
    uint32_t okA, okB;
    bool rA = produce(tA, okA), rB;
    // One exit, at the end of the loop body (an exit after every fold would
    // give the compiler paths that skip loads, and stricter load waits).
    if constexpr (NBUF == 2) {
      do {
        rB = produce(tB, okB);
        consume(rA, okA, tA);
        rA = produce(tA, okA);
        consume(rB, okB, tB);
      } while (has(kAlive));
    } else {
      Tile tC;
      uint32_t okC;
      bool rC;
      rB = produce(tB, okB);
      do {
        rC = produce(tC, okC);
        consume(rA, okA, tA);
        rA = produce(tA, okA);
        consume(rB, okB, tB);
        rB = produce(tB, okB);
        consume(rC, okC, tC);
      } while (has(kAlive));
    }
    return carry;
  };
  // Blocks shared between sequences (a common prefix) are likely to be read
  // again by other workgroups: keep the default cache policy for them.
  // Otherwise every K/V row is read once, and the loads are non-temporal --
  // except in vLLM's layout when a tile reads only part of every K group and V
  // row of its block (16-token tiles in blocks of 32 or more, 32-token tiles in
  // blocks of 64 or more) and the next tile reads the rest.  With the
  // shared-prefix hint, the shared units come first in the list: a wavefront
  // walks those at the default policy, then starts a second walk, non-temporal,
  // at its first private unit (one pipeline restart per wavefront, and no
  // branch inside the tile loop).  Without the hint, blocks found shared
  // between neighbours keep the default policy for every unit.
  {
    uint32_t t = share((uint32_t)wave);
    const bool all_default = (Vllm && prm.bs_log2 >= (TOK == 32 ? 6 : 5)) ||
                             (SPG == 0u && __builtin_amdgcn_readfirstlane(s_shared) != 0);
    const uint32_t default_end = all_default ? nunits : SPG * upp;
    if (t < default_end) t = walk(CachePolicy<0>{}, t, default_end);
    if (t < nunits) walk(CachePolicy<kAuxNT>{}, t, nunits);
  }
#ifdef PA_TIMELINE
  const uint64_t tl_exit = __builtin_amdgcn_s_memrealtime();
  const size_t wrec = (size_t)wg * NW + (size_t)wave;
  if (lane == 0 && 16 + 4 * wrec + 4 <= (size_t)kTlUnitBase) {
    uint64_t* r = g_timeline + 16 + 4 * wrec;
    r[0] = tl_entry;
    r[1] = tl_list;
    r[2] = tl_exit;
    // XCC_ID (hardware register 20), the wavefronts per workgroup, and HW_ID
    // (register 4)
    r[3] = (uint64_t)__builtin_amdgcn_s_getreg((4 << 11) | 20) | ((uint64_t)NW << 8) |
           ((uint64_t)__builtin_amdgcn_s_getreg((31 << 11) | 4) << 32);
  }
#endif
}

namespace {
constexpr int kMaxPersistentSeqs = 4096;   // the pair search covers 64 x 64 sequences
constexpr size_t kMinLdsPerCU = 82 * 1024; // more than half of a CU's 160 KiB of LDS

template <int D, bool WholeTile, int NW, bool Vllm, int TOK>
hipError_t launch_persistent(const DecodeParams& prm, int cus, hipStream_t stream) {
  // the list, padded so that a second workgroup never fits on the same CU
  size_t lds = (size_t)prm.B * 5 * sizeof(int32_t);
  const size_t fixed = sizeof(uint8_t) * NW * 2 * 16 * 2 * D + 64 * 4 + 12;
  if (lds + fixed < kMinLdsPerCU) lds = kMinLdsPerCU - fixed;
  hipLaunchKernelGGL((decode_partial_mfma_kernel<D, WholeTile, NW, Vllm, TOK>), dim3((uint32_t)cus), dim3(64 * NW),
                     lds, stream, prm);
  return hipGetLastError();
}

template <int D, bool WholeTile, bool Vllm>
hipError_t launch_mfma(const DecodeParams& prm, hipStream_t stream) {
  // Wavefronts per CU: two per SIMD while a wavefront needs at most half a
  // SIMD's registers (head_dim <= 128), else one.
  constexpr int NW = D <= 128 ? 8 : 4;
  const int cus = device_cus();
  if (prm.B <= kMaxPersistentSeqs && cus > 0) {
    if constexpr (Vllm && WholeTile && D <= 128) {
      // vLLM layout, blocks of 32 tokens or more: 32-token tiles, which hold
      // twice the registers of a 16-token tile (one wavefront per SIMD above
      // head_dim 64: the same bytes in flight per CU; at head_dim 256 they
      // would spill, so that size keeps 16-token tiles)
      if (prm.bs_log2 >= 5) return launch_persistent<D, true, D <= 64 ? 8 : 4, true, 32>(prm, cus, stream);
    }
    return launch_persistent<D, WholeTile, NW, Vllm, 16>(prm, cus, stream);
  }
  const dim3 grid(prm.KVH * prm.nchunks, prm.maxP, prm.B);
  if constexpr (Vllm)
    hipLaunchKernelGGL((decode_partial_vllm_kernel<D, WholeTile>), grid, dim3(64), 0, stream, prm);
  else
    hipLaunchKernelGGL((decode_partial_mfma_grid_kernel<D, WholeTile>), grid, dim3(64), 0, stream, prm);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_partials_mfma(const DecodeParams& prm, int32_t D, hipStream_t stream) {
  const bool whole = prm.bs_log2 >= 4;
  switch (D) {
    case 64: return whole ? launch_mfma<64, true, false>(prm, stream) : launch_mfma<64, false, false>(prm, stream);
    case 128: return whole ? launch_mfma<128, true, false>(prm, stream) : launch_mfma<128, false, false>(prm, stream);
    case 256: return whole ? launch_mfma<256, true, false>(prm, stream) : launch_mfma<256, false, false>(prm, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_partials_vllm(const DecodeParams& prm, int32_t D, hipStream_t stream) {
  const bool whole = prm.bs_log2 >= 4;
  switch (D) {
    case 64: return whole ? launch_mfma<64, true, true>(prm, stream) : launch_mfma<64, false, true>(prm, stream);
    case 128: return whole ? launch_mfma<128, true, true>(prm, stream) : launch_mfma<128, false, true>(prm, stream);
    case 256: return whole ? launch_mfma<256, true, true>(prm, stream) : launch_mfma<256, false, true>(prm, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
