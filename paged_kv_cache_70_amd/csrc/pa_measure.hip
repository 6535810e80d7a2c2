// Measurement helpers (not steps of the method), timed beside the kernels on
// the same device: a plain streaming read of a device buffer with 16-byte
// loads, the access width of the decode's KV gather, optionally non-temporal
// like the decode's loads (the ceiling a gather of the same byte count is
// measured against); and a run of independent bf16 matrix products with no
// memory traffic (the ceiling of the prefill's products).
#include "../../include/paged_kv.h"
#include "pa_internal.h"

namespace pa {

namespace {

typedef uint32_t u32x4r __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;   // independent 16-byte loads in flight per lane

// Workgroup w of G reads the w-th of G contiguous chunks of the buffer, 256
// threads side by side (4 KiB per round of one load each) and kReadUnroll
// loads in flight per lane, through a buffer resource over its chunk (loads
// past the chunk's end read zeros; aux 2 = non-temporal).  One contiguous
// stream per workgroup measured fastest of the access orders tried on
// MI355X (grid-strided 1 KiB pieces: 6% slower on 538 MB).  The loaded words
// are folded into an XOR that is stored only if it equals `tag`, a kernel
// argument the compiler cannot see through, so the loads stay live (sink is a
// valid word either way).
template <int AUX>
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const char* __restrict__ buf, uint64_t n16,
                                                                   uint32_t* __restrict__ sink, uint32_t tag) {
  const uint64_t chunk = (n16 + gridDim.x - 1) / gridDim.x;      // 16-byte units per workgroup
  const uint64_t lo = (uint64_t)blockIdx.x * chunk;
  const uint64_t hi = lo + chunk < n16 ? lo + chunk : n16;
  if (lo >= hi) return;
  const uint32_t cnt = (uint32_t)(hi - lo);                      // < 2^27 by the host check
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(buf + lo * 16), (short)0, (int)(cnt * 16u), 0x00020000);
  u32x4r acc = {0u, 0u, 0u, 0u};
  for (uint32_t i = threadIdx.x; i < cnt; i += kReadUnroll * kReadThreads) {
    u32x4r v[kReadUnroll];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k)
      v[k] = __builtin_bit_cast(u32x4r, __builtin_amdgcn_raw_buffer_load_b128(r, (i + k * kReadThreads) * 16u, 0, AUX));
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) acc ^= v[k];
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == tag) sink[0] = x;
}

// Matrix-core throughput: every wavefront runs `iters` rounds of 4
// independent v_mfma_f32_32x32x16_bf16 chains on register operands (no
// memory traffic).  The 32x32 product keeps its accumulators in place from
// one round to the next; the same loop written with 16x16x32 products comes
// out of the compiler with accumulator register moves between the products
// (tens of them per round), and measures the moves, not the matrix pipe.
// The accumulators are folded into a store guarded like the read's, so the
// products stay live.
constexpr int kMfmaChains = 4;
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, uint32_t* __restrict__ sink, uint32_t tag) {
  typedef __bf16 bf16x8m __attribute__((ext_vector_type(8)));
  typedef float f32x16m __attribute__((ext_vector_type(16)));
  const float x = (float)(threadIdx.x & 7) * 0.001f;
  bf16x8m a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(x + (float)i);
    b[i] = (__bf16)(x - (float)i);
  }
  f32x16m c[kMfmaChains];
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) c[k][j] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kMfmaChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  }
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc += c[k][j];
  const uint32_t y = __float_as_uint(acc);
  if (y == tag) sink[0] = y;
}

}  // namespace

}  // namespace pa

using namespace pa;

extern "C" int pa_measure_read(const void* buf, size_t bytes, int32_t workgroups_per_cu, int32_t nontemporal,
                               uint32_t* sink, void* stream) {
  if (!buf || !sink) return PA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return PA_ERR_ALIGN;
  if (bytes % 16 || workgroups_per_cu <= 0 || workgroups_per_cu > 64) return PA_ERR_SHAPE;
  if (bytes == 0) return PA_OK;
  const int cus = device_cus();
  if (cus <= 0) return PA_ERR_LAUNCH;
  const uint64_t groups = (uint64_t)cus * workgroups_per_cu;
  const uint64_t n16 = bytes / 16;
  // a workgroup's chunk is addressed by one buffer resource with 32-bit byte offsets
  if ((n16 + groups - 1) / groups >= (1ull << 27)) return PA_ERR_TOO_LARGE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const char* p = static_cast<const char*>(buf);
  if (nontemporal)
    hipLaunchKernelGGL((stream_read_kernel<2>), dim3((uint32_t)groups), dim3(kReadThreads), 0, s, p, n16, sink,
                       0x9E3779B9u);
  else
    hipLaunchKernelGGL((stream_read_kernel<0>), dim3((uint32_t)groups), dim3(kReadThreads), 0, s, p, n16, sink,
                       0x9E3779B9u);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

extern "C" int pa_measure_mfma(int32_t iters, int32_t workgroups_per_cu, uint32_t* sink, void* stream) {
  if (!sink) return PA_ERR_NULL;
  if (iters <= 0 || workgroups_per_cu <= 0 || workgroups_per_cu > 8) return PA_ERR_SHAPE;
  const int cus = device_cus();
  if (cus <= 0) return PA_ERR_LAUNCH;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((uint32_t)(cus * workgroups_per_cu)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, sink, 0x9E3779B9u);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
