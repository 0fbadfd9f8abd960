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
//   slot[i, c] (optional) = the position within row i of the first edge from that id,
//               16-bit when every row has at most 65535 edges, else 32-bit.
//   Empty rows: out = 0, arg = -1 (slot all ones).
//
// Forward (one launch over every row, the plan's row bins, like the attention forward):
//   reduce_fwd_main   hub chunks -> (value, index) partials; medium rows one wavefront each;
//                     light rows one G-lane group each (16 bytes of the row per lane, by
//                     structured buffer loads, or plain 64-bit loads for tables past 4 GiB)
//   reduce_fwd_merge  one wavefront per hub row folds its chunk partials with the same
//                     (value, index) rule (exact: the rule is a total order, so the merge
//                     order does not matter; it is fixed anyway)
// Backward, dx[arg[i, c], c] += dout[i, c], over the cached transpose (column bins by
// out-degree), so each source row is written once and no atomics are needed:
//   reduce_bwd_main   column j walks its destinations i (ascending) and gathers either
//                     arg[i] (4 bytes per element; a parallel edge lists i twice in a row
//                     and is counted once) or, cheaper, slot[i] (2 bytes per element),
//                     matched against the transpose entry's position in row i (csc_rel;
//                     only the first of parallel edges can match); where an element
//                     matches, dout[i] is gathered and added
//   reduce_bwd_merge  hub columns: ordered sums of chunk partials
// The message is the gathered row itself, so values are compared as stored (bf16 widens
// exactly to fp32) and out is written back bit-exact.
#include <climits>
#include <type_traits>

#include "ga_device.h"
#include "ga_internal.h"

namespace ga {
namespace {

constexpr int kNoArg = INT_MAX;  // id of an empty state: any real neighbour id is smaller
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Backward modes: match on arg (source ids) or on 16- / 32-bit slots (row positions).
enum { kMatchArg = 0, kMatchSlot16 = 2, kMatchSlot32 = 4 };

// SORTED: every row lists its neighbours by ascending id, so among equal values the
// smallest id is also the earliest edge; the state then orders by (value, edge index)
// alone and the id is read from the row at the end (fewer operations per element). Lane
// groups then visit a row's edges from last to first and take values at least as good:
// the last such take among equal values is the earliest edge, an initial -inf (max) or
// +inf (min) is taken like any value, and NaN (never >= or <=) never is.
template <typename T, int G, int OP, int U, bool SORTED = false>
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
    int id[VEC];   // winner's id (unused while SORTED: read from indices at the end)
    int pos[VEC];  // CSR edge index of the winner (first edge from that id); INT_MAX = none
  };

  __device__ __forceinline__ static void init(State& s) {
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      s.v[c] = OP == kReduceMax ? -INFINITY : INFINITY;
      s.id[c] = kNoArg;
      s.pos[c] = INT_MAX;
    }
  }

  // (v, j) beats (b, i): a strictly better value, or an equal value from a smaller id.
  // Non-short-circuit operators keep the rule branch-free (lane masks and selects).
  __device__ __forceinline__ static bool better(float v, int j, float b, int i) {
    const bool w = OP == kReduceMax ? v > b : v < b;
    return w | ((v == b) & (j < i));
  }
  // ... and between two edges from the same id (equal values), the earlier edge. With
  // sorted rows the edge index alone orders equal values.
  __device__ __forceinline__ static bool better3(float v, int j, int p, float b, int i, int q) {
    const bool w = OP == kReduceMax ? v > b : v < b;
    if constexpr (SORTED) return w | ((v == b) & (p < q));
    return better(v, j, b, i) | ((j == i) & (p < q));
  }

  // Edge k from source j (ok = the edge slot is in range). Unsorted rows: a lane group
  // visits a row's edges in increasing k, so an edge from an id already held is never
  // earlier and the two-way rule suffices. Sorted rows: edges arrive in decreasing k and
  // an equal value replaces the winner (see SORTED above).
  __device__ __forceinline__ static void fold(State& s, const float* x, int j, int k, bool ok) {
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      if constexpr (SORTED) {
        const bool t = ok & (OP == kReduceMax ? x[c] >= s.v[c] : x[c] <= s.v[c]);
        s.v[c] = t ? x[c] : s.v[c];
        s.pos[c] = t ? k : s.pos[c];
      } else {
        const bool t = ok & better(x[c], j, s.v[c], s.id[c]);
        s.v[c] = t ? x[c] : s.v[c];
        s.id[c] = t ? j : s.id[c];
        s.pos[c] = t ? k : s.pos[c];
      }
    }
  }

  // Edges [e0, e1) of a row through the state; NGS lane groups share the edges. The loop
  // counter runs forward; with SORTED it maps to the edges in reverse (k = e1 - 1 - (n - e0),
  // written so that no intermediate passes 2^31 when the row lies near the end of a graph
  // of 2^31 - 2^16 edges).
  __device__ __forceinline__ static int edge_of(int e0, int e1, int n) {
    return SORTED ? e1 - 1 - (n - e0) : n;
  }
  template <int NGS>
  __device__ __forceinline__ static void run(const RedArgs& a, int e0, int e1, int seg0, int gs,
                                             int r, State& s) {
    constexpr int L = NGS * G;
    const int lane = threadIdx.x & (kWave - 1);
    const rows_t Xd = node_rows(a.x, a.ld * int(sizeof(raw_t)), a.n);
    const raw_t* __restrict__ X = IO::R(a.x);
    for (int base = e0; base < e1; base += L) {
      const int nb = min(L, e1 - base);
      const int li = lane - seg0;
      // lanes past the batch's edges name node n, one record past the table, which a
      // structured buffer load reads as zeros without touching memory; with plain 64-bit
      // loads (no range check) they name the batch's first edge, of the same row. A step's
      // spare slots read those lanes or, where a step is longer than a batch, edges of the
      // same batch, and the fold skips them either way
      const int jb = ld_stream(a.indices + edge_of(e0, e1, base + (li < nb ? li : 0)));
      const int my_j = (li < nb || a.wide) ? jb : a.n;
      for (int t = 0; t < nb; t += NGS * U) {
        int jj[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int pos = t + u * NGS + gs;
          ok[u] = pos < nb;
          jj[u] = __builtin_amdgcn_ds_bpermute((seg0 + pos) << 2, my_j);
        }
        raw_t xr[U];
        auto gather = [&](auto wide) {
#pragma unroll
          for (int u = 0; u < U; ++u)
            xr[u] = ld_node<decltype(wide)::value>(Xd, X, jj[u], a.ld, r);
        };
        if (a.wide)
          gather(std::true_type{});
        else
          gather(std::false_type{});
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float xf[VEC];
          L16::unpack(xr[u], xf);
          fold(s, xf, jj[u], edge_of(e0, e1, base + t + u * NGS + gs), ok[u]);
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
        const int oi = SORTED ? 0 : __shfl_xor(s.id[c], off);
        const int op = __shfl_xor(s.pos[c], off);
        const bool t = better3(ov, oi, op, s.v[c], s.id[c], s.pos[c]);
        s.v[c] = t ? ov : s.v[c];
        if constexpr (!SORTED) s.id[c] = t ? oi : s.id[c];
        s.pos[c] = t ? op : s.pos[c];
      }
    }
  }

  // Store the row's result; row_start = indptr[row] (slot positions are row-relative).
  __device__ __forceinline__ static void write_row(const RedArgs& a, int row, int row_start,
                                                   int r, const State& s) {
    float o[VEC];
    int ar[VEC];
    unsigned sl[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      const bool empty = s.pos[c] == INT_MAX;
      o[c] = empty ? 0.f : s.v[c];
      if constexpr (SORTED)
        ar[c] = empty ? -1 : a.indices[s.pos[c]];
      else
        ar[c] = empty ? -1 : s.id[c];
      sl[c] = empty ? 0xffffffffu : static_cast<unsigned>(s.pos[c] - row_start);
    }
    const size_t e0 = static_cast<size_t>(row) * a.ld * VEC + r * VEC;  // element offset
    if (a.slot) {
      if (a.slot_bytes == 2) {
        unsigned w[VEC / 2];
#pragma unroll
        for (int k = 0; k < VEC / 2; ++k) w[k] = (sl[2 * k] & 0xffffu) | (sl[2 * k + 1] << 16);
        if constexpr (VEC == 8)
          st_stream(reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.slot) + e0),
                    u32x4{w[0], w[1], w[2], w[3]});
        else
          st_stream(reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.slot) + e0),
                    u32x2{w[0], w[1]});
      } else {
        u32x4* sp = reinterpret_cast<u32x4*>(static_cast<uint32_t*>(a.slot) + e0);
#pragma unroll
        for (int k = 0; k < VEC / 4; ++k)
          st_stream(sp + k, u32x4{sl[4 * k], sl[4 * k + 1], sl[4 * k + 2], sl[4 * k + 3]});
      }
    }
    st_stream(static_cast<raw_t*>(a.out) + static_cast<size_t>(row) * a.ld + r, L16::pack(o));
    u32x4* ap = reinterpret_cast<u32x4*>(a.arg + e0);
#pragma unroll
    for (int k = 0; k < VEC / 4; ++k)
      st_stream(ap + k, u32x4{static_cast<unsigned>(ar[4 * k]),
                              static_cast<unsigned>(ar[4 * k + 1]),
                              static_cast<unsigned>(ar[4 * k + 2]),
                              static_cast<unsigned>(ar[4 * k + 3])});
  }

  __device__ __forceinline__ static void st_int(int32_t* base, int r, const int* x) {
    u32x4* p = reinterpret_cast<u32x4*>(base + r * VEC);
#pragma unroll
    for (int k = 0; k < VEC / 4; ++k)
      st_stream(p + k, u32x4{static_cast<unsigned>(x[4 * k]), static_cast<unsigned>(x[4 * k + 1]),
                             static_cast<unsigned>(x[4 * k + 2]),
                             static_cast<unsigned>(x[4 * k + 3])});
  }

  // Chunk partials always carry the winner's id: the merge compares ids, since the chunks
  // of a row regrouped by an XCD split are not in id order (sorted rows track only the
  // edge, so the id is read back from the chunk's own, just-streamed, indices).
  __device__ __forceinline__ static void write_partial(const RedArgs& a, int chunk, int r,
                                                       const State& s) {
    const size_t c0 = static_cast<size_t>(chunk) * a.ld * VEC;  // partials span full rows
    IO::store_f32(a.ws_val + c0, r, s.v);
    if constexpr (SORTED) {
      int id[VEC];
#pragma unroll
      for (int c = 0; c < VEC; ++c) id[c] = s.pos[c] == INT_MAX ? kNoArg : a.indices[s.pos[c]];
      st_int(a.ws_idx + c0, r, id);
    } else {
      st_int(a.ws_idx + c0, r, s.id);
    }
    st_int(a.ws_pos + c0, r, s.pos);
  }

  __device__ __forceinline__ static void fold_partial(const RedArgs& a, int chunk, int r,
                                                      State& s) {
    const size_t c0 = static_cast<size_t>(chunk) * a.ld * VEC + r * VEC;
    const f32x4* vp = reinterpret_cast<const f32x4*>(a.ws_val + c0);
    const u32x4* ip = reinterpret_cast<const u32x4*>(a.ws_idx + c0);
    const u32x4* pp = reinterpret_cast<const u32x4*>(a.ws_pos + c0);
#pragma unroll
    for (int k = 0; k < VEC / 4; ++k) {
      const f32x4 v = ld_stream(vp + k);
      const u32x4 i = SORTED ? u32x4{} : ld_stream(ip + k);
      const u32x4 q4 = ld_stream(pp + k);
      const float vv[4] = {v.x, v.y, v.z, v.w};
      const int ii[4] = {static_cast<int>(i.x), static_cast<int>(i.y), static_cast<int>(i.z),
                         static_cast<int>(i.w)};
      const int qq[4] = {static_cast<int>(q4.x), static_cast<int>(q4.y), static_cast<int>(q4.z),
                         static_cast<int>(q4.w)};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 4 * k + q;
        const bool t = better3(vv[q], ii[q], qq[q], s.v[c], s.id[c], s.pos[c]);
        s.v[c] = t ? vv[q] : s.v[c];
        if constexpr (!SORTED) s.id[c] = t ? ii[q] : s.id[c];
        s.pos[c] = t ? qq[q] : s.pos[c];
      }
    }
  }

  // ---- backward over transpose columns ---------------------------------------------
  // The lane's VEC match keys of destination row i: arg ids, or slots (row positions).
  template <int MODE>
  __device__ __forceinline__ static void load_keys(const RedArgs& a, int i, int r,
                                                   unsigned* key) {
    const size_t e0 = static_cast<size_t>(i) * a.ld * VEC + r * VEC;
    if constexpr (MODE == kMatchSlot16) {
      const uint16_t* sp = static_cast<const uint16_t*>(a.slot_in) + e0;
      unsigned w[VEC / 2];
      if constexpr (VEC == 8) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(sp);
        w[0] = x.x;
        w[1] = x.y;
        w[2] = x.z;
        w[3] = x.w;
      } else {
        const u32x2 x = *reinterpret_cast<const u32x2*>(sp);
        w[0] = x.x;
        w[1] = x.y;
      }
#pragma unroll
      for (int k = 0; k < VEC / 2; ++k) {
        key[2 * k] = w[k] & 0xffffu;
        key[2 * k + 1] = w[k] >> 16;
      }
    } else {
      const u32x4* kp = reinterpret_cast<const u32x4*>(
          MODE == kMatchArg ? static_cast<const void*>(a.arg_in + e0)
                            : static_cast<const void*>(
                                  static_cast<const uint32_t*>(a.slot_in) + e0));
#pragma unroll
      for (int k = 0; k < VEC / 4; ++k) {
        const u32x4 x = kp[k];
        key[4 * k] = x.x;
        key[4 * k + 1] = x.y;
        key[4 * k + 2] = x.z;
        key[4 * k + 3] = x.w;
      }
    }
  }

  // Destinations [e0, e1) of column j (cs = the column's first position). An element of
  // destination i matches when its arg is j (arg mode; a repeated i, a parallel edge, is
  // skipped) or when its slot is this transpose entry's position in row i (slot modes).
  template <int NGS, int MODE>
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
      // arg mode: the previous destination of the column (-1 at its start; equal ids are
      // adjacent); slot modes: this entry's position within its CSR row
      int my_k;
      if constexpr (MODE == kMatchArg)
        my_k = (li < nb && p > cs) ? ld_stream(a.rowidx + p - 1) : -1;
      else
        my_k = (li < nb) ? ld_stream(a.csc_rel + p) : 0;
      for (int t = 0; t < nb; t += NGS * U) {
        int ii[U];
        unsigned want[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int pos = t + u * NGS + gs;
          const int src = seg0 + (pos < nb ? pos : t);
          ii[u] = __shfl(my_i, src);
          const int k = __shfl(my_k, src);  // every lane takes part in the shuffles
          if constexpr (MODE == kMatchArg) {
            ok[u] = pos < nb && k != ii[u];
            want[u] = static_cast<unsigned>(j);
          } else {
            ok[u] = pos < nb;
            want[u] = static_cast<unsigned>(k);
          }
        }
        unsigned key[U][VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) load_keys<MODE>(a, ii[u], r, key[u]);
        bool hit[U][VEC];
        bool any[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          any[u] = false;
#pragma unroll
          for (int c = 0; c < VEC; ++c) {
            hit[u][c] = ok[u] && key[u][c] == want[u];
            any[u] |= hit[u][c];
          }
        }
        raw_t dr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          dr[u] = raw_t{};
          if (any[u]) dr[u] = Do[static_cast<size_t>(ii[u]) * a.ld + r];
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

// The main kernels work on a feature slice of G lanes of a row of a.ld lanes, slices dealt
// to XCDs by slice_of (ga_device.h); each wave moves its pointers to its slice.
template <typename T, int G, int OP, int U, bool SORTED>
__global__ __launch_bounds__(kBlock) void reduce_fwd_main(RedArgs a0) {
  using K = Red<T, G, OP, U, SORTED>;
  using raw_t = typename K::raw_t;
  constexpr int NG = K::NG, VEC = K::VEC;
  const int lane = threadIdx.x & (kWave - 1);
  const SliceItem si = slice_of(a0.slices);
  const int item = si.item;
  const int so = si.slice * G;  // lanes before this slice
  RedArgs a = a0;
  a.x = static_cast<const raw_t*>(a0.x) + so;
  a.out = static_cast<raw_t*>(a0.out) + so;
  a.arg = a0.arg + so * VEC;
  if (a0.slot) a.slot = static_cast<char*>(a0.slot) + static_cast<size_t>(so) * VEC * a0.slot_bytes;
  if (a0.ws_val) {
    a.ws_val = a0.ws_val + so * VEC;
    a.ws_idx = a0.ws_idx + so * VEC;
    a.ws_pos = a0.ws_pos + so * VEC;
  }
  const int g = lane / G, r = lane % G;
  const DevBins& B = a.rows;
  typename K::State s;
  K::init(s);
  if (item < B.n_sched + B.n_medium) {
    int row, e0, e1, c = 0;
    const bool chunk = item < B.n_sched;
    if (chunk) {
      c = chunk_of(B, item);
      if (c < 0) return;  // unused slot of an XCD schedule
      row = B.chunk_row[c];
      e0 = B.chunk_begin[c];
      e1 = B.chunk_end[c];
    } else {
      row = B.medium[item - B.n_sched];
      e0 = a.indptr[row];
      e1 = a.indptr[row + 1];
    }
    K::template run<NG>(a, e0, e1, 0, g, r, s);
    K::template combine<NG>(s);
    if (g != 0) return;
    if (chunk)
      K::write_partial(a, c, r, s);
    else
      K::write_row(a, row, e0, r, s);
    return;
  }
  const int li = (item - B.n_sched - B.n_medium) * NG + g;
  if (li >= B.n_light) return;
  const int row = B.light[li];
  const int e0 = a.indptr[row];
  K::template run<1>(a, e0, a.indptr[row + 1], g * G, 0, r, s);
  K::write_row(a, row, e0, r, s);
}

// One wavefront per hub row: group g folds chunks c0+g, c0+g+NG, ..., then the butterfly,
// always by the full (value, id, edge) rule.
template <typename T, int G, int OP>
__global__ __launch_bounds__(kBlock) void reduce_fwd_merge(RedArgs a) {
  using K = Red<T, G, OP, 1, false>;
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
  if (g == 0) K::write_row(a, row, a.indptr[row], r, s);
}

template <typename T, int G, int U, int MODE>
__global__ __launch_bounds__(kBlock) void reduce_bwd_main(RedArgs a0) {
  using K = Red<T, G, kReduceMax, U>;
  using raw_t = typename K::raw_t;
  constexpr int NG = K::NG, VEC = K::VEC;
  const int lane = threadIdx.x & (kWave - 1);
  const SliceItem si = slice_of(a0.slices);
  const int item = si.item;
  const int so = si.slice * G;  // lanes before this slice
  RedArgs a = a0;
  if (a0.arg_in) a.arg_in = a0.arg_in + so * VEC;
  if (a0.slot_in)
    a.slot_in =
        static_cast<const char*>(a0.slot_in) + static_cast<size_t>(so) * VEC * a0.slot_bytes;
  a.dout = static_cast<const raw_t*>(a0.dout) + so;
  a.dx = static_cast<raw_t*>(a0.dx) + so;
  if (a0.ws_sum) a.ws_sum = a0.ws_sum + so * VEC;
  const int g = lane / G, r = lane % G;
  const DevBins& B = a.cols;
  typename K::acc_t s[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) s[c] = 0;
  if (item < B.n_sched + B.n_medium) {
    int col, e0, e1, c = 0;
    const bool chunk = item < B.n_sched;
    if (chunk) {
      c = chunk_of(B, item);
      if (c < 0) return;  // unused slot of an XCD schedule
      col = B.chunk_row[c];
      e0 = B.chunk_begin[c];
      e1 = B.chunk_end[c];
    } else {
      col = B.medium[item - B.n_sched];
      e0 = a.colptr[col];
      e1 = a.colptr[col + 1];
    }
    K::template run_cols<NG, MODE>(a, col, e0, e1, a.colptr[col], 0, g, r, s);
    K::template group_sum<NG>(s);
    if (g != 0) return;
    if (chunk)
      K::store_f32(a.ws_sum + static_cast<size_t>(c) * a.ld * VEC, r, s);
    else
      K::store(a.dx, col, r, s, 1.f, a.ld);
    return;
  }
  const int li = (item - B.n_sched - B.n_medium) * NG + g;
  if (li >= B.n_light) return;
  const int col = B.light[li];
  const int e0 = a.colptr[col], e1 = a.colptr[col + 1];
  K::template run_cols<1, MODE>(a, col, e0, e1, e0, g * G, 0, r, s);
  K::store(a.dx, col, r, s, 1.f, a.ld);
}

template <typename T, int G>
__global__ __launch_bounds__(kBlock) void reduce_bwd_merge(RedArgs a) {
  using K = Red<T, G, kReduceMax, 1>;
  constexpr int NG = K::NG, VEC = K::VEC;
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
  for (int c = c0 + g; c < c1; c += NG)
    K::add_f32(a.ws_sum + static_cast<size_t>(c) * a.ld * VEC, r, s);
  K::template group_sum<NG>(s);
  if (g == 0) K::store(a.dx, col, r, s, 1.f);
}

// Edges per step of the forward: 2 keeps the kernel at 52 VGPRs (bf16, 32-lane rows), eight
// waves per SIMD, whose loads hide each other's latency better than deeper unrolls at
// fewer waves (8 edges: 82 VGPRs, five waves).
constexpr int kUnrollRed = 2;
#ifndef GA_UNROLL_RED_BWD
#define GA_UNROLL_RED_BWD 4
#endif
constexpr int kUnrollRedBwd = GA_UNROLL_RED_BWD;

template <typename Kern>
int go(const char* name, Kern kernel, int64_t blocks, const RedArgs& a, void* stream,
       TimerHook hook) {
  if (blocks <= 0) return 0;
  if (hook) hook(name, stream, 1);
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), a);
  if (hook) hook(name, stream, 0);
  return static_cast<int>(hipGetLastError());
}

inline int64_t blocks_of(int64_t waves) { return (waves + kWavesPerBlock - 1) / kWavesPerBlock; }

// Main kernel on the slice geometry (G lanes per slice, a.slices slices).
template <typename T, int G>
int launch_main(bool backward, int op, const RedArgs& a, void* stream, TimerHook hook) {
  constexpr int NG = kWave / G;
  auto items_of = [](const DevBins& B) {
    return int64_t(B.n_sched) + B.n_medium + (int64_t(B.n_light) + NG - 1) / NG;
  };
  if (backward) {
    const int64_t b = slice_blocks(blocks_of(items_of(a.cols)), a.slices);
    if (items_of(a.cols) <= 0) return 0;
    if (!a.slot_in)
      return go("reduce_bwd_main", reduce_bwd_main<T, G, kUnrollRedBwd, kMatchArg>, b, a, stream,
                hook);
    if (a.slot_bytes == 2)
      return go("reduce_bwd_main", reduce_bwd_main<T, G, kUnrollRedBwd, kMatchSlot16>, b, a,
                stream, hook);
    return go("reduce_bwd_main", reduce_bwd_main<T, G, kUnrollRedBwd, kMatchSlot32>, b, a,
              stream, hook);
  }
  if (items_of(a.rows) <= 0) return 0;
  const int64_t b = slice_blocks(blocks_of(items_of(a.rows)), a.slices);
  if (op == kReduceMax)
    return a.rows_sorted
               ? go("reduce_fwd_main", reduce_fwd_main<T, G, kReduceMax, kUnrollRed, true>, b, a,
                    stream, hook)
               : go("reduce_fwd_main", reduce_fwd_main<T, G, kReduceMax, kUnrollRed, false>, b,
                    a, stream, hook);
  return a.rows_sorted
             ? go("reduce_fwd_main", reduce_fwd_main<T, G, kReduceMin, kUnrollRed, true>, b, a,
                  stream, hook)
             : go("reduce_fwd_main", reduce_fwd_main<T, G, kReduceMin, kUnrollRed, false>, b, a,
                  stream, hook);
}

// Hub merges on the full row geometry.
template <typename T, int G>
int launch_merge(bool backward, int op, const RedArgs& a, void* stream, TimerHook hook) {
  if (backward)
    return go("reduce_bwd_merge", reduce_bwd_merge<T, G>, blocks_of(a.cols.n_hub), a, stream,
              hook);
  const int64_t b = blocks_of(a.rows.n_hub);
  return op == kReduceMax
             ? go("reduce_fwd_merge", reduce_fwd_merge<T, G, kReduceMax>, b, a, stream, hook)
             : go("reduce_fwd_merge", reduce_fwd_merge<T, G, kReduceMin>, b, a, stream, hook);
}

template <typename T>
int launch_t(bool backward, int op, int G, const RedArgs& a, void* stream, TimerHook hook) {
  int e = -1;
  switch (G / a.slices) {
    case 4: e = launch_main<T, 4>(backward, op, a, stream, hook); break;
    case 8: e = launch_main<T, 8>(backward, op, a, stream, hook); break;
    case 16: e = launch_main<T, 16>(backward, op, a, stream, hook); break;
    case 32: e = launch_main<T, 32>(backward, op, a, stream, hook); break;
    case 64: e = launch_main<T, 64>(backward, op, a, stream, hook); break;
  }
  if (e) return e;
  switch (G) {
    case 4: return launch_merge<T, 4>(backward, op, a, stream, hook);
    case 8: return launch_merge<T, 8>(backward, op, a, stream, hook);
    case 16: return launch_merge<T, 16>(backward, op, a, stream, hook);
    case 32: return launch_merge<T, 32>(backward, op, a, stream, hook);
    case 64: return launch_merge<T, 64>(backward, op, a, stream, hook);
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
