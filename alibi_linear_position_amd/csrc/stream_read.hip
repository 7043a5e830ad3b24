// Plain streaming read of a device buffer: the practical HBM read rate against
// which the decode's bandwidth is read. Measurement tool only, not on the
// attention path.
//
// It reads the way the decode does: each workgroup streams one contiguous slab
// of the buffer (bytes / workgroups, 16-byte aligned), every thread keeps eight
// non-temporal 16-byte loads in flight, and consecutive lanes read consecutive
// chunks. Every chunk is read exactly once. A workgroup writes the XOR of all
// words it read to sink[workgroup], so the loads cannot be optimised away and
// the XOR of the sink equals the XOR of the buffer.
#include "device_common.h"
#include "launch.h"

namespace alibi {

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ p, long long n16,
                                                                   long long slab, uint32_t* __restrict__ sink) {
  constexpr int U = kReadUnroll;
  __shared__ uint32_t red[kReadThreads / 64];
  const int tid = threadIdx.x;
  const long long beg = (long long)blockIdx.x * slab;
  const long long end = beg + slab < n16 ? beg + slab : n16;
  u32x4 a = {0u, 0u, 0u, 0u};
  for (long long i = beg + tid; i < end; i += (long long)kReadThreads * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long j = i + (long long)u * kReadThreads;
      v[u] = j < end ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) a ^= v[u];
  }
  uint32_t x = a[0] ^ a[1] ^ a[2] ^ a[3];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= uint32_t(__shfl_xor(int(x), off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = x;
  __syncthreads();
  if (tid == 0) {
    uint32_t y = 0u;
#pragma unroll
    for (int w = 0; w < kReadThreads / 64; ++w) y ^= red[w];
    sink[blockIdx.x] = y;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* buf, long long bytes, uint32_t* sink, int workgroups, hipStream_t stream) {
  const long long n16 = bytes / 16;
  const long long slab = (n16 + workgroups - 1) / workgroups;
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(workgroups)), dim3(kReadThreads), 0, stream,
                     static_cast<const u32x4*>(buf), n16, slab, sink);
  return hipGetLastError();
}

}  // namespace alibi
