// Host planner: CSR validation, degree binning, hub chunking and the cached transpose.
//
// Degree-aware tiling follows "On Efficient Scaling of GNNs via IO-Aware Layers
// Implementations", Technical Summary > Methodology (reduction-based layers): nodes are
// partitioned by a degree threshold; low-degree ones take a feature-parallel kernel and
// high-degree ones are reduced as parallel edge chunks. Here there are three bins (light /
// medium / hub) and hub chunks merge without atomics. The transpose follows the same
// section's SpMM paragraph (transposed adjacency precomputed once for the backward).
//
// Everything is O(N + E) (or O(N log N) when one degree dwarfs N), runs once per graph, and
// is bit-exact by construction: no floating point, and the threaded transpose writes every
// entry where the sequential counting sort would.
#include <algorithm>
#include <climits>
#include <new>
#include <thread>

#include "ga_internal.h"

namespace ga {
namespace {

// Ids 0..n-1 ordered by degree descending, ties by ascending id: a stable counting sort on
// the degree, whose buckets take 4 bytes per possible degree, when the largest degree is
// at most about n; a stable comparison sort otherwise.
void order_by_degree(const std::vector<int32_t>& ptr, std::vector<int32_t>* order,
                     int64_t* max_deg) {
  const int64_t n = static_cast<int64_t>(ptr.size()) - 1;
  order->resize(static_cast<size_t>(n));
  int64_t mx = 0;
  for (int64_t i = 0; i < n; ++i) mx = std::max<int64_t>(mx, ptr[i + 1] - ptr[i]);
  *max_deg = mx;
  if (mx <= n + 1024) {
    std::vector<int32_t> start(static_cast<size_t>(mx) + 1, 0);  // start[d]: first slot of degree d
    for (int64_t i = 0; i < n; ++i) start[ptr[i + 1] - ptr[i]]++;
    int32_t at = 0;
    for (int64_t d = mx; d >= 0; --d) {
      const int32_t c = start[d];
      start[d] = at;
      at += c;
    }
    for (int64_t i = 0; i < n; ++i) (*order)[start[ptr[i + 1] - ptr[i]]++] = static_cast<int32_t>(i);
    return;
  }
  for (int64_t i = 0; i < n; ++i) (*order)[i] = static_cast<int32_t>(i);
  std::stable_sort(order->begin(), order->end(), [&](int32_t x, int32_t y) {
    return ptr[x + 1] - ptr[x] > ptr[y + 1] - ptr[y];
  });
}

// Rows of `ptr` binned by degree; each bin lists ids by degree descending, ties by id.
// A hub is a row above the hub threshold or, when split > 0, above split. Rows above split
// are regrouped in place: their entries of `key` (and of `comp`, when given, in step) are
// stably ordered by key mod kXcds, and each nonempty group is chunked on its own, so every
// chunk of such a row reads the sources of one partition. sched then deals the chunks to
// dispatch slots: a slot s runs in workgroup s / kWavesPerSlotBlock, and workgroup w lands
// on XCD w mod kXcds, so partition p's chunks go to slots of workgroups w = p (mod kXcds);
// chunks of unsplit hubs are dealt to the partitions in turn. Within a partition chunks
// run longest first (ties by chunk id); unused slots hold -1. sched stays empty when no
// row is split. Returns false when the work items (chunk slots, medium rows, light rows)
// would not fit the kernels' 32-bit item index (a schedule can be up to 8 times longer
// than the chunk list when one partition holds every chunk).
bool bin_by_degree(const std::vector<int32_t>& ptr, const ga_plan_opts& o, int32_t split,
                   std::vector<int32_t>* key, std::vector<int32_t>* comp, Bins* b,
                   int64_t* max_deg) {
  std::vector<int32_t> order;
  order_by_degree(ptr, &order, max_deg);
  auto deg = [&](int32_t i) { return ptr[i + 1] - ptr[i]; };
  auto is_split = [&](int32_t d) { return split > 0 && d > split; };
  b->light.clear();
  b->medium.clear();
  b->hub.clear();
  for (int32_t i : order) {
    const int32_t d = deg(i);
    if (d <= o.light_max_deg)
      b->light.push_back(i);
    else if (d <= o.hub_min_deg_exclusive && !is_split(d))
      b->medium.push_back(i);
    else
      b->hub.push_back(i);
  }
  b->chunk_row.clear();
  b->chunk_begin.clear();
  b->chunk_end.clear();
  b->sched.clear();
  b->hub_chunk_ptr.assign(1, 0);
  std::vector<int32_t> tk, tc;
  std::vector<int8_t> part;  // per chunk: its partition, or -1 (unsplit hub)
  auto cut = [&](int32_t row, int64_t beg, int64_t end, int8_t p) {
    for (int64_t s = beg; s < end; s += o.hub_chunk) {
      b->chunk_row.push_back(row);
      b->chunk_begin.push_back(static_cast<int32_t>(s));
      b->chunk_end.push_back(static_cast<int32_t>(std::min<int64_t>(s + o.hub_chunk, end)));
      part.push_back(p);
    }
  };
  for (int32_t i : b->hub) {
    const int64_t beg = ptr[i], end = ptr[i + 1];
    if (!is_split(deg(i))) {
      cut(i, beg, end, -1);
    } else {
      int64_t at[kXcds + 1] = {0};
      for (int64_t k = beg; k < end; ++k) at[((*key)[k] & (kXcds - 1)) + 1]++;
      for (int p = 0; p < kXcds; ++p) at[p + 1] += at[p];
      const int64_t n = end - beg;
      tk.resize(static_cast<size_t>(n));
      if (comp) tc.resize(static_cast<size_t>(n));
      int64_t fill[kXcds];
      for (int p = 0; p < kXcds; ++p) fill[p] = at[p];
      for (int64_t k = beg; k < end; ++k) {
        const int64_t t = fill[(*key)[k] & (kXcds - 1)]++;
        tk[t] = (*key)[k];
        if (comp) tc[t] = (*comp)[k];
      }
      std::copy(tk.begin(), tk.end(), key->begin() + beg);
      if (comp) std::copy(tc.begin(), tc.end(), comp->begin() + beg);
      for (int p = 0; p < kXcds; ++p) cut(i, beg + at[p], beg + at[p + 1], static_cast<int8_t>(p));
    }
    b->hub_chunk_ptr.push_back(static_cast<int32_t>(b->chunk_row.size()));
  }
  const size_t rest = b->medium.size() + b->light.size();
  auto fits = [&](size_t slots) { return slots + rest <= size_t(INT32_MAX); };
  if (std::find_if(part.begin(), part.end(), [](int8_t p) { return p >= 0; }) == part.end())
    return fits(part.size());
  std::vector<int32_t> q[kXcds];
  int64_t turn = 0;
  for (size_t c = 0; c < part.size(); ++c)
    q[part[c] >= 0 ? part[c] : (turn++ % kXcds)].push_back(static_cast<int32_t>(c));
  size_t blocks = 0;
  for (auto& v : q) {
    std::stable_sort(v.begin(), v.end(), [&](int32_t x, int32_t y) {
      return b->chunk_end[x] - b->chunk_begin[x] > b->chunk_end[y] - b->chunk_begin[y];
    });
    blocks = std::max(blocks, (v.size() + kWavesPerSlotBlock - 1) / kWavesPerSlotBlock);
  }
  if (!fits(blocks * kXcds * kWavesPerSlotBlock)) return false;
  b->sched.assign(blocks * kXcds * kWavesPerSlotBlock, -1);
  for (int p = 0; p < kXcds; ++p)
    for (size_t k = 0; k < q[p].size(); ++k)
      b->sched[((k / kWavesPerSlotBlock) * kXcds + p) * kWavesPerSlotBlock +
               k % kWavesPerSlotBlock] = q[p][k];
  return true;
}

// Threads for the transpose: up to 16, one when the graph is small; fewer when the
// per-thread column counters (threads x N int32) would pass 1 GiB.
int transpose_threads(int64_t n, int64_t e) {
  if (e < (int64_t(1) << 16)) return 1;
  const unsigned hw = std::thread::hardware_concurrency();
  int t = hw ? static_cast<int>(std::min(hw, 16u)) : 1;
  while (t > 1 && int64_t(t) * n * 4 > (int64_t(1) << 30)) t /= 2;
  return t;
}

// Stable counting-sort transpose: colptr, and for every transpose entry its destination
// row and its position within that row; destinations ascend within each column. Rows are
// split into T contiguous blocks of about E/T edges. Block t counts its edges per column,
// then writes them, in row order, from the column's start plus the counts of blocks before
// it: the positions a single pass over the rows in order would use.
void transpose(const std::vector<int32_t>& indptr, const std::vector<int32_t>& indices,
               int64_t n, int64_t e, int T, std::vector<int32_t>* colptr,
               std::vector<int32_t>* rowidx, std::vector<int32_t>* rel,
               std::vector<int32_t>* cursor) {
  std::vector<int64_t> rb(static_cast<size_t>(T) + 1, n);  // block t: rows [rb[t], rb[t+1])
  rb[0] = 0;
  for (int t = 1; t < T; ++t)
    rb[t] = std::lower_bound(indptr.begin(), indptr.end(), static_cast<int32_t>(e * t / T)) -
            indptr.begin();
  for (int t = 1; t <= T; ++t) rb[t] = std::max(rb[t], rb[t - 1]);
  rb[T] = n;
  int32_t* cnt = cursor->data();  // [T][n]
  // blocks 1..T-1 on their own threads, block 0 here; a block whose thread cannot be
  // started runs here too (no exception leaves the planner)
  auto run = [&](auto&& body) {
    std::vector<std::thread> th;
    th.reserve(static_cast<size_t>(T));
    int t = 1;
    try {
      for (; t < T; ++t) th.emplace_back(body, t);
    } catch (...) {
    }
    for (int u = t; u < T; ++u) body(u);
    body(0);
    for (auto& x : th) x.join();
  };
  run([&](int t) {
    int32_t* c = cnt + static_cast<size_t>(t) * n;
    for (int64_t k = indptr[rb[t]]; k < indptr[rb[t + 1]]; ++k) c[indices[k]]++;
  });
  (*colptr)[0] = 0;
  for (int64_t j = 0; j < n; ++j) {
    int64_t at = (*colptr)[j];
    for (int t = 0; t < T; ++t) {
      int32_t& c = cnt[static_cast<size_t>(t) * n + j];
      const int32_t k = c;
      c = static_cast<int32_t>(at);  // block t's first slot in column j
      at += k;
    }
    (*colptr)[j + 1] = static_cast<int32_t>(at);
  }
  run([&](int t) {
    int32_t* c = cnt + static_cast<size_t>(t) * n;
    for (int64_t i = rb[t]; i < rb[t + 1]; ++i)
      for (int32_t k = indptr[i]; k < indptr[i + 1]; ++k) {
        const int32_t at = c[indices[k]]++;
        (*rowidx)[at] = static_cast<int32_t>(i);
        (*rel)[at] = k - indptr[i];  // the edge's position within its CSR row
      }
  });
}

}  // namespace

// Hub thresholds and chunks left at -1 are chosen from the graph's size. A hub row is
// split so that no single wavefront holds much more than its share of the edges: with
// about 8192 wavefronts in flight on the GPU, rows longer than E / 8192 edges (rounded to
// the nearest power of two, kept within [256, 8192]) become chunked hubs, in chunks of a
// quarter of that (at least 256). Column passes do more work per edge and keep smaller
// hubs (at most 1024, chunks at most 512).
ga_plan_opts resolve_opts(const ga_plan_opts& in, int64_t e) {
  ga_plan_opts o = in;
  if (o.hub_min_deg_exclusive == -1) {
    const double share = static_cast<double>(e) / 8192.0;
    int64_t t = 256;
    while (t < 8192 && static_cast<double>(t) * 1.4142135623730951 < share) t *= 2;
    o.hub_min_deg_exclusive = static_cast<int32_t>(std::max<int64_t>(t, o.light_max_deg));
  }
  if (o.hub_chunk == -1) o.hub_chunk = std::max(256, o.hub_min_deg_exclusive / 4);
  if (o.col_hub_min_deg_exclusive == -1)
    o.col_hub_min_deg_exclusive = std::max(std::min(1024, o.hub_min_deg_exclusive),
                                           o.light_max_deg);
  if (o.col_hub_chunk == -1) o.col_hub_chunk = std::min(512, o.hub_chunk);
  return o;
}

ga_status build_plan(const int32_t* indptr, const int32_t* indices, int64_t n, int64_t e,
                     const ga_plan_opts& given, ga_plan* p) {
  // Kernels step through edge positions in 32-bit integers, up to 64 past a row's end
  // before the loop test: E keeps 2^16 of headroom below 2^31.
  if (n < 0 || e < 0 || n >= (int64_t(1) << 31) || e > kMaxEdges) return GA_ERR_INVALID_ARG;
  if (!indptr || (e > 0 && !indices)) return GA_ERR_INVALID_ARG;
  if (given.light_max_deg < 0 || given.hub_min_deg_exclusive < -1 || given.hub_chunk < -1 ||
      given.hub_chunk == 0 || given.col_hub_min_deg_exclusive < -1 ||
      given.col_hub_chunk < -1 || given.col_hub_chunk == 0 ||
      given.xcd_split_min_deg_exclusive < 0 || given.col_xcd_split_min_deg_exclusive < 0 ||
      (given.xcd_split_min_deg_exclusive > 0 &&
       given.xcd_split_min_deg_exclusive < given.light_max_deg) ||
      (given.col_xcd_split_min_deg_exclusive > 0 &&
       given.col_xcd_split_min_deg_exclusive < given.light_max_deg))
    return GA_ERR_INVALID_ARG;
  const ga_plan_opts o = resolve_opts(given, e);
  if (o.hub_min_deg_exclusive < o.light_max_deg || o.col_hub_min_deg_exclusive < o.light_max_deg)
    return GA_ERR_INVALID_ARG;
  if (o.feature_slices != 0 && o.feature_slices != 1 && o.feature_slices != 2 &&
      o.feature_slices != 4 && o.feature_slices != 8)
    return GA_ERR_INVALID_ARG;
  // validation
  if (indptr[0] != 0 || indptr[n] != e) return GA_ERR_BAD_GRAPH;
  for (int64_t i = 0; i < n; ++i)
    if (indptr[i + 1] < indptr[i]) return GA_ERR_BAD_GRAPH;
  for (int64_t k = 0; k < e; ++k)
    if (indices[k] < 0 || indices[k] >= n) return GA_ERR_BAD_GRAPH;

  try {
    p->n = n;
    p->e = e;
    p->opts = o;
    p->indptr.assign(indptr, indptr + n + 1);
    p->indices.assign(indices, indices + e);
    p->rows_sorted = true;
    for (int64_t i = 0; i < n && p->rows_sorted; ++i)
      for (int32_t k = indptr[i] + 1; k < indptr[i + 1]; ++k)
        if (indices[k] < indices[k - 1]) {
          p->rows_sorted = false;
          break;
        }
    // regroups split rows of p->indices; the transpose below is of that CSR
    if (!bin_by_degree(p->indptr, o, o.xcd_split_min_deg_exclusive, &p->indices, nullptr,
                       &p->rows, &p->max_in))
      return GA_ERR_UNSUPPORTED;
    p->has_csc = o.build_csc != 0;
    p->max_out = 0;
    if (p->has_csc) {
      const int T = transpose_threads(n, e);
      p->colptr.assign(static_cast<size_t>(n) + 1, 0);
      p->rowidx.assign(static_cast<size_t>(e), 0);
      p->csc_rel.assign(static_cast<size_t>(e), 0);
      std::vector<int32_t> cursor(static_cast<size_t>(T) * static_cast<size_t>(n), 0);
      transpose(p->indptr, p->indices, n, e, T, &p->colptr, &p->rowidx, &p->csc_rel, &cursor);
      ga_plan_opts oc = o;  // the transpose's columns use their own hub threshold / chunk
      oc.hub_min_deg_exclusive = o.col_hub_min_deg_exclusive;
      oc.hub_chunk = o.col_hub_chunk;
      if (!bin_by_degree(p->colptr, oc, o.col_xcd_split_min_deg_exclusive, &p->rowidx,
                         &p->csc_rel, &p->cols, &p->max_out))
        return GA_ERR_UNSUPPORTED;
    } else {
      p->colptr.clear();
      p->rowidx.clear();
      p->csc_rel.clear();
      p->cols = Bins{};
    }
  } catch (const std::bad_alloc&) {
    return GA_ERR_HOST_ALLOC;
  }
  p->uploaded = false;
  return GA_OK;
}

}  // namespace ga
