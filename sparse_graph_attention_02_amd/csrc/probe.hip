// Streaming copy kernel: measures achievable HBM copy bandwidth on the device and gives a
// kernel of exactly known traffic (bytes read = bytes written = n) for calibrating the
// TCC read/write byte counters.
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {
namespace {

constexpr int kCopyUnroll = 4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kBlock) void copy_probe(u32x4* __restrict__ dst,
                                                     const u32x4* __restrict__ src, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kBlock;
  size_t i = static_cast<size_t>(blockIdx.x) * kBlock + threadIdx.x;
  for (; i + (kCopyUnroll - 1) * stride < n16; i += kCopyUnroll * stride) {
    u32x4 x[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) x[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(x[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

int launch_copy(void* dst, const void* src, size_t bytes, void* stream, TimerHook hook) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return 0;
  // enough blocks to fill 256 CUs several times over, each thread streaming 4 x 16 bytes
  size_t blocks = (n16 + kBlock * kCopyUnroll - 1) / (kBlock * kCopyUnroll);
  if (blocks > 256 * 64) blocks = 256 * 64;
  if (hook) hook("copy_probe", stream, 1);
  hipLaunchKernelGGL(copy_probe, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4*>(dst),
                     static_cast<const u32x4*>(src), n16);
  if (hook) hook("copy_probe", stream, 0);
  return static_cast<int>(hipGetLastError());
}

}  // namespace ga
