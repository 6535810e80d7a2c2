// Measurement helper (not a step of the method): a plain streaming read of a
// device buffer with 16-byte loads, the access width of the decode's KV
// gather, optionally non-temporal like the decode's loads.  Timed beside the
// decode on the same box, its rate is the ceiling a gather of the same byte
// count is measured against.
#include "../../include/paged_kv.h"
#include "pa_internal.h"

namespace pa {

namespace {

typedef uint32_t u32x4r __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;   // independent 16-byte loads in flight per lane

// Thread t reads 16-byte units t, t + S, t + 2 S, ... (S = all threads of the
// grid), kReadUnroll at a time; one instruction of a wavefront covers 1 KiB
// of contiguous bytes.  The loaded words are folded into an XOR that is
// stored only if it equals `tag`, a kernel argument the compiler cannot see
// through, so the loads stay live (sink is a valid word either way).
template <bool NT>
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4r* __restrict__ buf, uint64_t n16,
                                                                   uint32_t* __restrict__ sink, uint32_t tag) {
  const uint64_t stride = (uint64_t)gridDim.x * kReadThreads;
  uint64_t i = (uint64_t)blockIdx.x * kReadThreads + threadIdx.x;
  u32x4r acc = {0u, 0u, 0u, 0u};
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4r v[kReadUnroll];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k)
      v[k] = NT ? __builtin_nontemporal_load(buf + i + k * stride) : buf[i + k * stride];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) acc ^= v[k];
  }
  for (; i < n16; i += stride) acc ^= NT ? __builtin_nontemporal_load(buf + i) : buf[i];
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == tag) sink[0] = x;
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
  const dim3 grid((uint32_t)(cus * workgroups_per_cu));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4r* p = static_cast<const u32x4r*>(buf);
  if (nontemporal)
    hipLaunchKernelGGL((stream_read_kernel<true>), grid, dim3(kReadThreads), 0, s, p, (uint64_t)(bytes / 16), sink,
                       0x9E3779B9u);
  else
    hipLaunchKernelGGL((stream_read_kernel<false>), grid, dim3(kReadThreads), 0, s, p, (uint64_t)(bytes / 16), sink,
                       0x9E3779B9u);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
