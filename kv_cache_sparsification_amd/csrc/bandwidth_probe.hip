// Measurement probes.
//
// Streaming read: the rate at which one plain kernel reads device memory on this chip.
//
// The memory-bound steps of the path (compaction, paged decode) are reported against the
// published HBM peak; this kernel gives the practical ceiling beside it: 16 bytes per lane
// per load, four independent loads in flight per lane, a grid-stride walk over the buffer,
// nontemporal loads (the data is read once).  Each workgroup folds what it read into one
// word and stores it only if it matches a value the caller passes, so the loads cannot be
// dropped and the kernel writes (almost) nothing.
#include "kvs_common.h"

namespace kvs {
namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 4;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                               uint32_t key, uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t folded = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (folded == key) sink[blockIdx.x] = folded;
}

// Clock stamp: one lane stores the GPU's fixed-frequency real-time counter (100 MHz on this
// chip).  Placed as the first and last nodes of a captured graph, two stamps time the work
// between them from when the graph starts running, without the latency of starting it.
__global__ __launch_bounds__(kWave) void timestamp_kernel(uint64_t* __restrict__ out) {
  const uint64_t t = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) out[0] = t;
}

}  // namespace
}  // namespace kvs

using namespace kvs;

extern "C" int kvs_probe_stream_read(const void* buf, size_t bytes, int grid, uint32_t key, uint32_t* sink,
                                     void* stream) {
  if (!buf || !sink) return fail(KVS_E_INVAL, "kvs_probe_stream_read: NULL pointer");
  if (bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15))
    return fail(KVS_E_INVAL, "kvs_probe_stream_read: bytes must be a positive multiple of 16, buf 16-byte aligned");
  if (grid < 1 || grid > (1 << 20)) return fail(KVS_E_INVAL, "kvs_probe_stream_read: grid out of range");
  stream_read_kernel<<<grid, kThreads, 0, as_stream(stream)>>>(static_cast<const u32x4*>(buf), bytes / 16, key,
                                                               sink);
  return launch_status("kvs_probe_stream_read");
}

extern "C" int kvs_probe_timestamp(uint64_t* out, void* stream) {
  if (!out || (reinterpret_cast<uintptr_t>(out) & 7))
    return fail(KVS_E_INVAL, "kvs_probe_timestamp: out must be a non-NULL, 8-byte aligned device pointer");
  timestamp_kernel<<<1, kWave, 0, as_stream(stream)>>>(out);
  return launch_status("kvs_probe_timestamp");
}
