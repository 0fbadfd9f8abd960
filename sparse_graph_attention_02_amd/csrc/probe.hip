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
  for (; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Gather-only pass over a CSR: for every edge, the G lanes of a group load the 16-byte
// slices of the source's K and V rows (the forward's gather pattern: 64 / G edges per wave
// step, U = 8 steps in flight), with no arithmetic beyond an XOR that keeps the loads live.
// Its time is the memory system's floor for the forward's neighbour gathers on that graph.
template <int G>
__global__ __launch_bounds__(kBlock) void gather_probe(const int32_t* __restrict__ indices,
                                                      int64_t e,
                                                       const u32x4* __restrict__ K,
                                                       const u32x4* __restrict__ V, u32x4* sink) {
  constexpr int NG = kWave / G, U = 8;
  const int lane = threadIdx.x & (kWave - 1), g = lane / G, r = lane % G;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  const int64_t base = wave * NG * U;
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t ed = base + u * NG + g;
    if (ed < e) {
      const int j = __builtin_nontemporal_load(indices + ed);
      acc ^= K[static_cast<size_t>(j) * G + r] ^ V[static_cast<size_t>(j) * G + r];
    }
  }
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) sink[lane] = acc;  // practically never
}

}  // namespace

int launch_gather_probe(const int32_t* indices, int64_t e, int G, const void* k, const void* v,
                        void* sink, void* stream, TimerHook hook) {
  if (e == 0) return 0;
  const int64_t per_wave = (kWave / G) * 8;
  const int64_t blocks = ((e + per_wave - 1) / per_wave + kWavesPerBlock - 1) / kWavesPerBlock;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* K = static_cast<const u32x4*>(k);
  const u32x4* V = static_cast<const u32x4*>(v);
  u32x4* out = static_cast<u32x4*>(sink);
  if (hook) hook("gather_probe", stream, 1);
  switch (G) {
#define GA_G(GG)                                                                          \
  case GG:                                                                                \
    hipLaunchKernelGGL(gather_probe<GG>, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s, \
                       indices, e, K, V, out);                                            \
    break;
    GA_G(4) GA_G(8) GA_G(16) GA_G(32) GA_G(64)
#undef GA_G
    default:
      return -1;
  }
  if (hook) hook("gather_probe", stream, 0);
  return static_cast<int>(hipGetLastError());
}

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
