// Measurement kernels. A streaming copy kernel measures achievable HBM copy bandwidth and
// gives a kernel of exactly known traffic (bytes read = bytes written = n) for calibrating
// the TCC read/write byte counters; gather-only probes measure the memory floor of the
// attention passes' access patterns on a plan, and a random-row gather over a table of
// chosen size measures the gather ceiling of the memory hierarchy at that footprint.
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {
namespace {

constexpr int kCopyUnroll = 4;

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

// Gather-only probes: the memory traffic of a pass with its arithmetic taken out. Each
// loads what the pass it stands beside loads, in the same order, with the same lanes
// (16 bytes per lane, G lanes per row), the same work items and index batches, and folds
// the loaded words into an XOR that keeps the loads live; none writes anything but an
// improbable sink store. Every item keeps 8 edges in flight per lane group, at least as
// many as the passes (a pass with fewer, and arithmetic between its loads, measured no
// faster than a probe with 8). Their durations are floors for those passes' times on the
// same graph and plan: what the memory system takes to deliver their reads.
struct ProbeArgs {
  const int32_t* ptr;     // indptr (rows) or colptr (columns)
  const int32_t* idx;     // indices (rows) or rowidx (columns)
  DevBins bins;           // row or column bins (with the plan's XCD schedule)
  const u32x4* side_a;    // per-item operand rows read once per work item (null: none)
  const u32x4* side_b;
  const u32x4* gx;        // rows gathered per edge (gy null: one row per edge)
  const u32x4* gy;
  const f32x2* rec;       // per-edge (lse, D) record per head (columns; null: none)
  u32x4* sink;
  int ld;                 // feature row stride in lanes (the full row)
  int heads;              // record stride (heads per node)
  int lh_shift;           // log2(lanes per head)
  int slices;             // feature slices (rows probe)
};

__device__ __forceinline__ void probe_sink(const ProbeArgs& a, const u32x4& acc, int lane) {
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x2545f491u)
    a.sink[lane] = acc;  // practically never
}

// Edges [e0, e1) of one work item, NGS lane groups cooperating (the attention passes'
// index batch: one index per lane, broadcast by shuffles, U edges per group per step;
// masked slots re-read the step's first edge, as the dQ and column passes do; the
// buffer-fed passes give them a record past the table instead, which loads nothing, so
// there the probe's masked slots are L2 hits the pass does not make).
template <int G, int U, int NGS, bool COLS>
__device__ __forceinline__ void probe_edges(const ProbeArgs& a, int e0, int e1, int seg0, int gs,
                                            int r, int h, u32x4& acc) {
  constexpr int L = NGS * G;
  const int lane = threadIdx.x & (kWave - 1);
  for (int base = e0; base < e1; base += L) {
    const int nb = min(L, e1 - base);
    const int li = lane - seg0;
    const int my = (li < nb) ? ld_stream(a.idx + base + li) : 0;
    for (int t = 0; t < nb; t += NGS * U) {
      int jj[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pos = t + u * NGS + gs;
        jj[u] = __shfl(my, seg0 + (pos < nb ? pos : t));
      }
      u32x4 x[U], y[U];
      f32x2 z[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t row = static_cast<size_t>(jj[u]);
        x[u] = a.gx[row * a.ld + r];
        if (a.gy) y[u] = a.gy[row * a.ld + r];
        if (COLS && a.rec) z[u] = a.rec[row * a.heads + h];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        acc ^= x[u];
        if (a.gy) acc ^= y[u];
        if (COLS && a.rec) {
          acc.x ^= __float_as_uint(z[u].x);
          acc.y ^= __float_as_uint(z[u].y);
        }
      }
    }
  }
}

// The work list of the forward and the dQ pass (rows), or of the dK/dV pass (columns):
// [0, n_sched) chunk slots (the plan's XCD schedule, -1 = unused), then medium items (one
// wavefront each), then light items (one G-lane group each). Rows run in feature slices
// as the forward does.
template <int G, int U, int UL, bool COLS>
__device__ __forceinline__ void probe_items(const ProbeArgs& a0) {
  constexpr int NG = kWave / G;
  const int lane = threadIdx.x & (kWave - 1);
  const SliceItem si = slice_of(a0.slices);
  const int item = si.item;
  ProbeArgs a = a0;
  const int so = si.slice * G;  // lanes before this slice
  a.gx = a0.gx + so;
  if (a0.gy) a.gy = a0.gy + so;
  if (a0.side_a) a.side_a = a0.side_a + so;
  if (a0.side_b) a.side_b = a0.side_b + so;
  const int g = lane / G, r = lane % G, h = r >> a.lh_shift;
  const DevBins& B = a.bins;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int node, e0, e1;
  bool wide;
  if (item < B.n_sched + B.n_medium) {
    wide = true;
    if (item < B.n_sched) {
      const int c = chunk_of(B, item);
      if (c < 0) return;  // unused slot of an XCD schedule
      node = B.chunk_row[c];
      e0 = B.chunk_begin[c];
      e1 = B.chunk_end[c];
    } else {
      node = B.medium[item - B.n_sched];
      e0 = a.ptr[node];
      e1 = a.ptr[node + 1];
    }
  } else {
    wide = false;
    const int li = (item - B.n_sched - B.n_medium) * NG + g;
    if (li >= B.n_light) return;
    node = B.light[li];
    e0 = a.ptr[node];
    e1 = a.ptr[node + 1];
  }
  const size_t off = static_cast<size_t>(node) * a.ld + r;
  if (a.side_a) acc ^= ld_stream(a.side_a + off);
  if (a.side_b) acc ^= ld_stream(a.side_b + off);
  if (wide)
    probe_edges<G, U, NG, COLS>(a, e0, e1, 0, g, r, h, acc);
  else
    probe_edges<G, UL, 1, COLS>(a, e0, e1, g * G, 0, r, h, acc);
  probe_sink(a, acc, lane);
}

constexpr int kProbeUnroll = 8;

template <int G>
__global__ __launch_bounds__(kBlock) void gather_probe_rows(ProbeArgs a) {
  probe_items<G, kProbeUnroll, kProbeUnroll, false>(a);
}

template <int G>
__global__ __launch_bounds__(kBlock) void gather_probe_cols(ProbeArgs a) {
  probe_items<G, kProbeUnroll, kProbeUnroll, true>(a);
}

// Uniformly random rows of a table: gather k of a launch reads row
// floor(hi32(x_k) * rows / 2^32), x_k = mix(seed + k * 0x9e3779b97f4a7c15), the k-th output
// of the SplitMix64 generator (Steele, Lea and Flood, OOPSLA 2014: a Weyl sequence through
// its output mixing function). G lanes per row, U rows in flight per lane group.
__device__ __forceinline__ uint64_t splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

template <int G, int U>
__global__ __launch_bounds__(kBlock) void gather_probe_random(const u32x4* __restrict__ table,
                                                              uint32_t rows, int64_t n,
                                                              uint64_t seed, u32x4* sink) {
  constexpr int NG = kWave / G;
  const int lane = threadIdx.x & (kWave - 1), g = lane / G, r = lane % G;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  const int64_t base = wave * NG * U;
  u32x4 x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t k = base + u * NG + g;
    const uint64_t m = splitmix64_mix(seed + static_cast<uint64_t>(k) * 0x9e3779b97f4a7c15ull);
    const uint32_t row = static_cast<uint32_t>(((m >> 32) * rows) >> 32);
    x[u] = k < n ? table[static_cast<size_t>(row) * G + r] : u32x4{0u, 0u, 0u, 0u};
  }
  u32x4 acc = x[0];
#pragma unroll
  for (int u = 1; u < U; ++u) acc ^= x[u];
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x2545f491u) sink[lane] = acc;
}

}  // namespace

namespace {

template <bool COLS>
int launch_items(const ProbeLaunch& p, void* stream, TimerHook hook) {
  ProbeArgs a{};
  a.ptr = p.ptr;
  a.idx = p.idx;
  a.bins = p.bins;
  a.side_a = static_cast<const u32x4*>(p.side_a);
  a.side_b = static_cast<const u32x4*>(p.side_b);
  a.gx = static_cast<const u32x4*>(p.gx);
  a.gy = static_cast<const u32x4*>(p.gy);
  a.rec = static_cast<const f32x2*>(p.rec);
  a.sink = static_cast<u32x4*>(p.sink);
  a.ld = p.G;
  a.heads = p.heads;
  a.lh_shift = 0;
  while ((1 << a.lh_shift) < p.LH) ++a.lh_shift;
  a.slices = COLS ? 1 : p.slices;
  const int GS = p.G / a.slices;
  const int NG = kWave / GS;
  const DevBins& B = p.bins;
  const int64_t items = int64_t(B.n_sched) + B.n_medium + (int64_t(B.n_light) + NG - 1) / NG;
  if (items <= 0) return 0;
  const int64_t blocks = slice_blocks((items + kWavesPerBlock - 1) / kWavesPerBlock, a.slices);
  const char* name = COLS ? "gather_probe_cols" : "gather_probe_rows";
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hook) hook(name, stream, 1);
  switch (GS) {
#define GA_G(GG)                                                                        \
  case GG:                                                                              \
    if (COLS)                                                                           \
      hipLaunchKernelGGL((gather_probe_cols<GG>),                                       \
                         dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s, a);   \
    else                                                                                \
      hipLaunchKernelGGL((gather_probe_rows<GG>),                                       \
                         dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s, a);   \
    break;
    GA_G(4) GA_G(8) GA_G(16) GA_G(32) GA_G(64)
#undef GA_G
    default:
      return -1;
  }
  if (hook) hook(name, stream, 0);
  return static_cast<int>(hipGetLastError());
}
}  // namespace

int launch_gather_probe_rows(const ProbeLaunch& p, void* stream, TimerHook hook) {
  return launch_items<false>(p, stream, hook);
}

int launch_gather_probe_cols(const ProbeLaunch& p, void* stream, TimerHook hook) {
  return launch_items<true>(p, stream, hook);
}

int launch_gather_probe_random(int G, const void* table, int64_t rows, int64_t n, uint64_t seed,
                               void* sink, void* stream, TimerHook hook) {
  if (n <= 0) return 0;
  const int64_t per_wave = (kWave / G) * kProbeUnroll;
  const int64_t blocks = ((n + per_wave - 1) / per_wave + kWavesPerBlock - 1) / kWavesPerBlock;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* T = static_cast<const u32x4*>(table);
  u32x4* out = static_cast<u32x4*>(sink);
  const uint32_t r = static_cast<uint32_t>(rows);
  if (hook) hook("gather_probe_random", stream, 1);
  switch (G) {
#define GA_G(GG)                                                                          \
  case GG:                                                                                \
    hipLaunchKernelGGL((gather_probe_random<GG, kProbeUnroll>),                           \
                       dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s, T, r, n, seed, \
                       out);                                                              \
    break;
    GA_G(4) GA_G(8) GA_G(16) GA_G(32) GA_G(64)
#undef GA_G
    default:
      return -1;
  }
  if (hook) hook("gather_probe_random", stream, 0);
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
