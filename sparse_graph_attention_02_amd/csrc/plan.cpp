// Host planner: CSR validation, degree binning, hub chunking and the cached transpose.
//
// Degree-aware tiling follows "On Efficient Scaling of GNNs via IO-Aware Layers
// Implementations", Technical Summary > Methodology (reduction-based layers): nodes are
// partitioned by a degree threshold; low-degree ones take a feature-parallel kernel and
// high-degree ones are reduced as parallel edge chunks. Here there are three bins (light /
// medium / hub) and hub chunks merge without atomics. The transpose follows the same
// section's SpMM paragraph (transposed adjacency precomputed once for the backward).
//
// Everything is O(N + E) or O(N log N), runs once per graph, and is bit-exact by
// construction (no floating point, no parallel reordering).
#include <algorithm>
#include <new>

#include "ga_internal.h"

namespace ga {
namespace {

// Rows of `ptr` binned by degree; each bin lists ids by degree descending, ties by id.
void bin_by_degree(const std::vector<int32_t>& ptr, const ga_plan_opts& o, Bins* b,
                   int64_t* max_deg) {
  const int64_t n = static_cast<int64_t>(ptr.size()) - 1;
  std::vector<int32_t> order(static_cast<size_t>(n));
  for (int64_t i = 0; i < n; ++i) order[i] = static_cast<int32_t>(i);
  auto deg = [&](int32_t i) { return ptr[i + 1] - ptr[i]; };
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t x, int32_t y) { return deg(x) > deg(y); });
  b->light.clear();
  b->medium.clear();
  b->hub.clear();
  *max_deg = 0;
  for (int32_t i : order) {
    const int32_t d = deg(i);
    if (d > *max_deg) *max_deg = d;
    if (d <= o.light_max_deg)
      b->light.push_back(i);
    else if (d <= o.hub_min_deg_exclusive)
      b->medium.push_back(i);
    else
      b->hub.push_back(i);
  }
  b->chunk_row.clear();
  b->chunk_begin.clear();
  b->chunk_end.clear();
  b->hub_chunk_ptr.assign(1, 0);
  for (int32_t i : b->hub) {
    const int64_t beg = ptr[i], end = ptr[i + 1];
    for (int64_t s = beg; s < end; s += o.hub_chunk) {
      b->chunk_row.push_back(i);
      b->chunk_begin.push_back(static_cast<int32_t>(s));
      b->chunk_end.push_back(static_cast<int32_t>(std::min<int64_t>(s + o.hub_chunk, end)));
    }
    b->hub_chunk_ptr.push_back(static_cast<int32_t>(b->chunk_row.size()));
  }
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
  if (n < 0 || e < 0 || n >= (int64_t(1) << 31) || e >= (int64_t(1) << 31))
    return GA_ERR_INVALID_ARG;
  if (!indptr || (e > 0 && !indices)) return GA_ERR_INVALID_ARG;
  if (given.light_max_deg < 0 || given.hub_min_deg_exclusive < -1 || given.hub_chunk < -1 ||
      given.hub_chunk == 0 || given.col_hub_min_deg_exclusive < -1 ||
      given.col_hub_chunk < -1 || given.col_hub_chunk == 0)
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
    bin_by_degree(p->indptr, o, &p->rows, &p->max_in);
    p->rows_sorted = true;
    for (int64_t i = 0; i < n && p->rows_sorted; ++i)
      for (int32_t k = indptr[i] + 1; k < indptr[i + 1]; ++k)
        if (indices[k] < indices[k - 1]) {
          p->rows_sorted = false;
          break;
        }
    p->has_csc = o.build_csc != 0;
    p->max_out = 0;
    if (p->has_csc) {
      // stable counting-sort transpose: scanning rows in order leaves destinations
      // ascending inside every column
      p->colptr.assign(static_cast<size_t>(n) + 1, 0);
      for (int64_t k = 0; k < e; ++k) p->colptr[indices[k] + 1]++;
      for (int64_t j = 0; j < n; ++j) p->colptr[j + 1] += p->colptr[j];
      std::vector<int32_t> cursor(p->colptr.begin(), p->colptr.end() - 1);
      p->rowidx.assign(static_cast<size_t>(e), 0);
      p->csc_rel.assign(static_cast<size_t>(e), 0);
      for (int64_t i = 0; i < n; ++i)
        for (int32_t k = indptr[i]; k < indptr[i + 1]; ++k) {
          const int32_t at = cursor[indices[k]]++;
          p->rowidx[at] = static_cast<int32_t>(i);
          p->csc_rel[at] = k - indptr[i];  // the edge's position within its CSR row
        }
      ga_plan_opts oc = o;  // the transpose's columns use their own hub threshold / chunk
      oc.hub_min_deg_exclusive = o.col_hub_min_deg_exclusive;
      oc.hub_chunk = o.col_hub_chunk;
      bin_by_degree(p->colptr, oc, &p->cols, &p->max_out);
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
