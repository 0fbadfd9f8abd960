// Degree-aware neighbourhood reduction (min / max pooling) for gfx950.
//
// Method: "On Efficient Scaling of GNNs via IO-Aware Layers Implementations", Technical
// Summary > Methodology, reduction-based layers: a per-edge message reduced over each
// node's neighbourhood (min / max pooling), with degree-aware tiling: light rows are
// handled feature-parallel, heavy rows as parallel edge chunks whose partial results are
// combined as (value, index) pairs.
//
//   out[i, c] = max_j x[j, c] (or min) over the neighbours j of row i,
//   arg[i, c] = the source id attaining it; equal values go to the smallest id, so the
//               result does not depend on neighbour order or on how a row is split.
//   Empty rows: out = 0, arg = -1.
//
// Forward (one launch over every row, the plan's row bins, like the attention forward):
//   reduce_fwd_main   hub chunks -> (value, index) partials; medium rows one wavefront each;
//                     light rows one G-lane group each (16 bytes of the row per lane)
//   reduce_fwd_merge  one wavefront per hub row folds its chunk partials with the same
//                     (value, index) rule (exact: the rule is a total order, so the merge
//                     order does not matter; it is fixed anyway)
// Backward, dx[arg[i, c], c] += dout[i, c], over the cached transpose (column bins by
// out-degree), so each source row is written once and no atomics are needed:
//   reduce_bwd_main   column j walks its destinations i (ascending; a parallel edge lists i
//                     twice in a row and is counted once), gathers arg[i] and, in the
//                     lanes where some element's arg is j, dout[i]
//   reduce_bwd_merge  hub columns: ordered sums of chunk partials
// The message is the gathered row itself, so values are compared as stored (bf16 widens
// exactly to fp32) and out is written back bit-exact.
#include <climits>

#include "ga_device.h"
#include "ga_internal.h"

namespace ga {
namespace {

constexpr int kNoArg = INT_MAX;  // id of an empty state: any real neighbour id is smaller

template <typename T, int G, int OP, int U>
struct Red : RowIO<T, G, G> {
  using IO = RowIO<T, G, G>;
  using typename IO::L16;
  using typename IO::raw_t;
  using IO::F;
  using IO::NG;
  using IO::VEC;
  using typename IO::acc_t;

  struct State {
    float v[VEC];
    int id[VEC];
  };

  __device__ __forceinline__ static void init(State& s) {
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      s.v[c] = OP == kReduceMax ? -INFINITY : INFINITY;
      s.id[c] = kNoArg;
    }
  }

  // (v, j) beats (b, i): a strictly better value, or an equal value from a smaller id.
  __device__ __forceinline__ static bool better(float v, int j, float b, int i) {
    const bool w = OP == kReduceMax ? v > b : v < b;
    return w || (v == b && j < i);
  }

  __device__ __forceinline__ static void fold(State& s, const float* x, int j) {
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      const bool t = better(x[c], j, s.v[c], s.id[c]);
      s.v[c] = t ? x[c] : s.v[c];
      s.id[c] = t ? j : s.id[c];
    }
  }

  // Edges [e0, e1) of a row through the state; NGS lane groups share the edges.
  template <int NGS>
  __device__ __forceinline__ static void run(const RedArgs& a, int e0, int e1, int seg0, int gs,
                                             int r, State& s) {
    constexpr int L = NGS * G;
    const int lane = threadIdx.x & (kWave - 1);
    const raw_t* __restrict__ X = IO::R(a.x);
    for (int base = e0; base < e1; base += L) {
      const int nb = min(L, e1 - base);
      const int li = lane - seg0;
      const int my_j = (li < nb) ? ld_stream(a.indices + base + li) : 0;
      for (int t = 0; t < nb; t += NGS * U) {
        int jj[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int pos = t + u * NGS + gs;
          ok[u] = pos < nb;
          // out-of-range slots re-read this step's first edge (valid) and are skipped
          jj[u] = __shfl(my_j, seg0 + (ok[u] ? pos : t));
        }
        raw_t xr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) xr[u] = X[static_cast<size_t>(jj[u]) * G + r];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (!ok[u]) continue;
          float xf[VEC];
          L16::unpack(xr[u], xf);
          fold(s, xf, jj[u]);
        }
      }
    }
  }

  // Fold the states of the NGS lane groups of a segment (butterfly; every lane ends with
  // the winner, which is unique, so the result does not depend on the pairing).
  template <int NGS>
  __device__ __forceinline__ static void combine(State& s) {
#pragma unroll
    for (int off = G; off < NGS * G; off <<= 1) {
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        const float ov = __shfl_xor(s.v[c], off);
        const int oi = __shfl_xor(s.id[c], off);
        const bool t = better(ov, oi, s.v[c], s.id[c]);
        s.v[c] = t ? ov : s.v[c];
        s.id[c] = t ? oi : s.id[c];
      }
    }
  }

  __device__ __forceinline__ static void write_row(const RedArgs& a, int row, int r,
                                                   const State& s) {
    float o[VEC];
    int ar[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      const bool empty = s.id[c] == kNoArg;
      o[c] = empty ? 0.f : s.v[c];
      ar[c] = empty ? -1 : s.id[c];
    }
    st_stream(static_cast<raw_t*>(a.out) + static_cast<size_t>(row) * G + r, L16::pack(o));
    u32x4* ap = reinterpret_cast<u32x4*>(a.arg + static_cast<size_t>(row) * F + r * VEC);
#pragma unroll
    for (int k = 0; k < VEC / 4; ++k)
      st_stream(ap + k, u32x4{static_cast<unsigned>(ar[4 * k]), static_cast<unsigned>(ar[4 * k + 1]),
                              static_cast<unsigned>(ar[4 * k + 2]),
                              static_cast<unsigned>(ar[4 * k + 3])});
  }

  __device__ __forceinline__ static void write_partial(const RedArgs& a, int chunk, int r,
                                                       const State& s) {
    IO::store_f32(a.ws_val + static_cast<size_t>(chunk) * F, r, s.v);
    u32x4* ip = reinterpret_cast<u32x4*>(a.ws_idx + static_cast<size_t>(chunk) * F + r * VEC);
#pragma unroll
    for (int k = 0; k < VEC / 4; ++k)
      st_stream(ip + k, u32x4{static_cast<unsigned>(s.id[4 * k]),
                              static_cast<unsigned>(s.id[4 * k + 1]),
                              static_cast<unsigned>(s.id[4 * k + 2]),
                              static_cast<unsigned>(s.id[4 * k + 3])});
  }

  __device__ __forceinline__ static void fold_partial(const RedArgs& a, int chunk, int r,
                                                      State& s) {
    const f32x4* vp =
        reinterpret_cast<const f32x4*>(a.ws_val + static_cast<size_t>(chunk) * F + r * VEC);
    const u32x4* ip =
        reinterpret_cast<const u32x4*>(a.ws_idx + static_cast<size_t>(chunk) * F + r * VEC);
#pragma unroll
    for (int k = 0; k < VEC / 4; ++k) {
      const f32x4 v = ld_stream(vp + k);
      const u32x4 i = ld_stream(ip + k);
      const float vv[4] = {v.x, v.y, v.z, v.w};
      const int ii[4] = {static_cast<int>(i.x), static_cast<int>(i.y), static_cast<int>(i.z),
                         static_cast<int>(i.w)};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 4 * k + q;
        const bool t = better(vv[q], ii[q], s.v[c], s.id[c]);
        s.v[c] = t ? vv[q] : s.v[c];
        s.id[c] = t ? ii[q] : s.id[c];
      }
    }
  }

  // ---- backward over transpose columns ---------------------------------------------
  // Destinations [e0, e1) of column j (cs = the column's first position, for the
  // duplicate test across a chunk boundary).
  template <int NGS>
  __device__ __forceinline__ static void run_cols(const RedArgs& a, int j, int e0, int e1,
                                                  int cs, int seg0, int gs, int r, acc_t* s) {
    constexpr int L = NGS * G;
    const int lane = threadIdx.x & (kWave - 1);
    const raw_t* __restrict__ Do = IO::R(a.dout);
    for (int base = e0; base < e1; base += L) {
      const int nb = min(L, e1 - base);
      const int li = lane - seg0;
      const int p = base + li;
      const int my_i = (li < nb) ? ld_stream(a.rowidx + p) : 0;
      // previous destination of the column (-1 at its start): equal ids are adjacent
      const int my_prev = (li < nb && p > cs) ? ld_stream(a.rowidx + p - 1) : -1;
      for (int t = 0; t < nb; t += NGS * U) {
        int ii[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int pos = t + u * NGS + gs;
          const int src = seg0 + (pos < nb ? pos : t);
          ii[u] = __shfl(my_i, src);
          const int prev = __shfl(my_prev, src);  // every lane takes part in the shuffle
          ok[u] = pos < nb && prev != ii[u];
        }
        u32x4 ar[U][VEC / 4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const u32x4* ap =
              reinterpret_cast<const u32x4*>(a.arg_in + static_cast<size_t>(ii[u]) * F + r * VEC);
#pragma unroll
          for (int k = 0; k < VEC / 4; ++k) ar[u][k] = ap[k];
        }
        bool hit[U][VEC];
        bool any[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          any[u] = false;
#pragma unroll
          for (int k = 0; k < VEC / 4; ++k) {
            const unsigned w[4] = {ar[u][k].x, ar[u][k].y, ar[u][k].z, ar[u][k].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              hit[u][4 * k + q] = ok[u] && static_cast<int>(w[q]) == j;
              any[u] |= hit[u][4 * k + q];
            }
          }
        }
        raw_t dr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          dr[u] = raw_t{};
          if (any[u]) dr[u] = Do[static_cast<size_t>(ii[u]) * G + r];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (!any[u]) continue;
          float df[VEC];
          L16::unpack(dr[u], df);
#pragma unroll
          for (int c = 0; c < VEC; ++c)
            if (hit[u][c]) s[c] += static_cast<acc_t>(df[c]);
        }
      }
    }
  }
};

template <typename T, int G, int OP, int U>
__global__ __launch_bounds__(kBlock) void reduce_fwd_main(RedArgs a) {
  using K = Red<T, G, OP, U>;
  constexpr int NG = K::NG;
  const int lane = threadIdx.x & (kWave - 1);
  const int item = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int g = lane / G, r = lane % G;
  const DevBins& B = a.rows;
  typename K::State s;
  K::init(s);
  if (item < B.n_chunks + B.n_medium) {
    int row, e0, e1;
    const bool chunk = item < B.n_chunks;
    if (chunk) {
      row = B.chunk_row[item];
      e0 = B.chunk_begin[item];
      e1 = B.chunk_end[item];
    } else {
      row = B.medium[item - B.n_chunks];
      e0 = a.indptr[row];
      e1 = a.indptr[row + 1];
    }
    K::template run<NG>(a, e0, e1, 0, g, r, s);
    K::template combine<NG>(s);
    if (g != 0) return;
    if (chunk)
      K::write_partial(a, item, r, s);
    else
      K::write_row(a, row, r, s);
    return;
  }
  const int li = (item - B.n_chunks - B.n_medium) * NG + g;
  if (li >= B.n_light) return;
  const int row = B.light[li];
  K::template run<1>(a, a.indptr[row], a.indptr[row + 1], g * G, 0, r, s);
  K::write_row(a, row, r, s);
}

// One wavefront per hub row: group g folds chunks c0+g, c0+g+NG, ..., then the butterfly.
template <typename T, int G, int OP>
__global__ __launch_bounds__(kBlock) void reduce_fwd_merge(RedArgs a) {
  using K = Red<T, G, OP, 1>;
  constexpr int NG = K::NG;
  const int hub = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane / G, r = lane % G;
  if (hub >= a.rows.n_hub) return;
  const int row = a.rows.hub[hub];
  const int c0 = a.rows.hub_chunk_ptr[hub], c1 = a.rows.hub_chunk_ptr[hub + 1];
  typename K::State s;
  K::init(s);
#pragma unroll 4
  for (int c = c0 + g; c < c1; c += NG) K::fold_partial(a, c, r, s);
  K::template combine<NG>(s);
  if (g == 0) K::write_row(a, row, r, s);
}

template <typename T, int G, int U>
__global__ __launch_bounds__(kBlock) void reduce_bwd_main(RedArgs a) {
  using K = Red<T, G, kReduceMax, U>;
  constexpr int NG = K::NG, VEC = K::VEC, F = K::F;
  const int lane = threadIdx.x & (kWave - 1);
  const int item = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int g = lane / G, r = lane % G;
  const DevBins& B = a.cols;
  typename K::acc_t s[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) s[c] = 0;
  if (item < B.n_chunks + B.n_medium) {
    int col, e0, e1;
    const bool chunk = item < B.n_chunks;
    if (chunk) {
      col = B.chunk_row[item];
      e0 = B.chunk_begin[item];
      e1 = B.chunk_end[item];
    } else {
      col = B.medium[item - B.n_chunks];
      e0 = a.colptr[col];
      e1 = a.colptr[col + 1];
    }
    K::template run_cols<NG>(a, col, e0, e1, a.colptr[col], 0, g, r, s);
    K::template group_sum<NG>(s);
    if (g != 0) return;
    if (chunk)
      K::store_f32(a.ws_sum + static_cast<size_t>(item) * F, r, s);
    else
      K::store(a.dx, col, r, s, 1.f);
    return;
  }
  const int li = (item - B.n_chunks - B.n_medium) * NG + g;
  if (li >= B.n_light) return;
  const int col = B.light[li];
  const int e0 = a.colptr[col], e1 = a.colptr[col + 1];
  K::template run_cols<1>(a, col, e0, e1, e0, g * G, 0, r, s);
  K::store(a.dx, col, r, s, 1.f);
}

template <typename T, int G>
__global__ __launch_bounds__(kBlock) void reduce_bwd_merge(RedArgs a) {
  using K = Red<T, G, kReduceMax, 1>;
  constexpr int NG = K::NG, VEC = K::VEC, F = K::F;
  const int hub = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane / G, r = lane % G;
  if (hub >= a.cols.n_hub) return;
  const int col = a.cols.hub[hub];
  const int c0 = a.cols.hub_chunk_ptr[hub], c1 = a.cols.hub_chunk_ptr[hub + 1];
  typename K::acc_t s[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) s[c] = 0;
#pragma unroll 4
  for (int c = c0 + g; c < c1; c += NG) K::add_f32(a.ws_sum + static_cast<size_t>(c) * F, r, s);
  K::template group_sum<NG>(s);
  if (g == 0) K::store(a.dx, col, r, s, 1.f);
}

constexpr int kUnrollRed = 8;
constexpr int kUnrollRedBwd = 4;

template <typename T, int G>
int launch_g(bool backward, int op, const RedArgs& a, void* stream, TimerHook hook) {
  constexpr int NG = kWave / G;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto items_of = [](const DevBins& B) {
    return int64_t(B.n_chunks) + B.n_medium + (int64_t(B.n_light) + NG - 1) / NG;
  };
  auto go = [&](const char* name, auto kernel, int64_t waves) -> int {
    const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks <= 0) return 0;
    if (hook) hook(name, stream, 1);
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s, a);
    if (hook) hook(name, stream, 0);
    return static_cast<int>(hipGetLastError());
  };
  int e;
  if (backward) {
    if ((e = go("reduce_bwd_main", reduce_bwd_main<T, G, kUnrollRedBwd>, items_of(a.cols))))
      return e;
    return go("reduce_bwd_merge", reduce_bwd_merge<T, G>, a.cols.n_hub);
  }
  if (op == kReduceMax) {
    if ((e = go("reduce_fwd_main", reduce_fwd_main<T, G, kReduceMax, kUnrollRed>,
                items_of(a.rows))))
      return e;
    return go("reduce_fwd_merge", reduce_fwd_merge<T, G, kReduceMax>, a.rows.n_hub);
  }
  if ((e = go("reduce_fwd_main", reduce_fwd_main<T, G, kReduceMin, kUnrollRed>,
              items_of(a.rows))))
    return e;
  return go("reduce_fwd_merge", reduce_fwd_merge<T, G, kReduceMin>, a.rows.n_hub);
}

template <typename T>
int launch_t(bool backward, int op, int G, const RedArgs& a, void* stream, TimerHook hook) {
  switch (G) {
    case 4: return launch_g<T, 4>(backward, op, a, stream, hook);
    case 8: return launch_g<T, 8>(backward, op, a, stream, hook);
    case 16: return launch_g<T, 16>(backward, op, a, stream, hook);
    case 32: return launch_g<T, 32>(backward, op, a, stream, hook);
    case 64: return launch_g<T, 64>(backward, op, a, stream, hook);
  }
  return -1;
}

}  // namespace

bool reduce_supported(ga_dtype dt, int G) {
  return (dt == GA_F32 || dt == GA_BF16) && (G == 4 || G == 8 || G == 16 || G == 32 || G == 64);
}

int launch_reduce(ga_dtype dt, bool backward, int op, int G, const RedArgs& a, void* stream,
                  TimerHook hook) {
  return dt == GA_F32 ? launch_t<float>(backward, op, G, a, stream, hook)
                      : launch_t<bf16_t>(backward, op, G, a, stream, hook);
}

}  // namespace ga
