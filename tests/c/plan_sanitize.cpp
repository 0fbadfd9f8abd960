// Host driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of the planner and
// the plan entry points of the C ABI (graph_attn_plan_*): seeded random graphs under many
// option sets, the degenerate graphs, and invalid CSR input. Every array a plan exports is
// read element by element, so an out-of-bounds write or read inside the planner shows up
// under the sanitizers; a few cheap invariants are checked on the way. Exit status 0 and
// no sanitizer report is a pass.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "graph_attn.h"

static int failures = 0;
#define CHECK(cond, ...)                          \
  do {                                            \
    if (!(cond)) {                                \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);          \
      std::fprintf(stderr, "\n");                 \
      ++failures;                                 \
    }                                             \
  } while (0)

struct Csr {
  std::vector<int32_t> ptr, idx;
  int64_t n() const { return int64_t(ptr.size()) - 1; }
};

// Degrees: mostly small, a tail of medium rows, a few hubs; sources uniform (parallel
// edges allowed), each row sorted or left in draw order.
static Csr random_graph(std::mt19937_64& rng, int64_t n, int hubs, int hub_deg, bool sorted) {
  Csr g;
  g.ptr.assign(n + 1, 0);
  std::geometric_distribution<int> small(0.15);
  std::uniform_int_distribution<int64_t> node(0, n > 0 ? n - 1 : 0);
  std::vector<int> deg(n);
  for (int64_t i = 0; i < n; ++i) deg[i] = (rng() % 10 == 0) ? 20 + int(rng() % 400) : small(rng);
  for (int h = 0; h < hubs && n > 0; ++h) deg[node(rng)] = hub_deg;
  for (int64_t i = 0; i < n; ++i) g.ptr[i + 1] = g.ptr[i] + deg[i];
  g.idx.resize(g.ptr[n]);
  for (int64_t i = 0; i < n; ++i) {
    for (int32_t e = g.ptr[i]; e < g.ptr[i + 1]; ++e) g.idx[e] = int32_t(node(rng));
    if (sorted) std::sort(g.idx.begin() + g.ptr[i], g.idx.begin() + g.ptr[i + 1]);
  }
  return g;
}

// Build a plan, read every exported array in full, check a few invariants, destroy it.
static void exercise(const Csr& g, const ga_plan_opts& o, const char* tag) {
  ga_plan* p = nullptr;
  const ga_status st = graph_attn_plan_create(g.ptr.data(), g.idx.data(), g.n(),
                                              int64_t(g.idx.size()), &o, &p);
  CHECK(st == GA_OK, "%s: plan_create returned %s", tag, graph_attn_status_string(st));
  if (st != GA_OK) return;
  ga_plan_info info;
  CHECK(graph_attn_plan_get_info(p, &info) == GA_OK, "%s: get_info", tag);
  size_t bytes = 0;
  CHECK(graph_attn_plan_device_bytes(p, &bytes) == GA_OK, "%s: device_bytes", tag);
  CHECK(info.n_nodes == g.n() && info.n_edges == int64_t(g.idx.size()), "%s: counts", tag);
  CHECK(info.n_row_light + info.n_row_medium + info.n_row_hub == g.n(), "%s: row bins", tag);
  int64_t touched = 0, sum = 0;
  for (int32_t k = 0; k < graph_attn_plan_array_count(); ++k) {
    const char* name = graph_attn_plan_array_name(k);
    CHECK(name != nullptr, "%s: array name %d", tag, k);
    if (!name) continue;
    const int32_t* data = nullptr;
    int64_t count = -1;
    const ga_status s = graph_attn_plan_array(p, name, &data, &count);
    if (s != GA_OK) {  // transpose arrays of a plan built without it
      CHECK(!info.has_csc, "%s: array %s missing: %s", tag, name, graph_attn_status_string(s));
      continue;
    }
    CHECK(count >= 0 && (count == 0 || data != nullptr), "%s: array %s", tag, name);
    for (int64_t i = 0; i < count; ++i) sum += data[i];
    touched += count;
    const std::string nm(name);
    if (nm == "indptr" || nm == "colptr") {
      CHECK(count == g.n() + 1, "%s: %s length", tag, name);
      if (count == g.n() + 1) CHECK(data[g.n()] == int32_t(g.idx.size()), "%s: %s end", tag, name);
      for (int64_t i = 0; i + 1 < count; ++i)
        if (data[i] > data[i + 1]) {
          CHECK(false, "%s: %s not monotone at %lld", tag, name, (long long)i);
          break;
        }
    }
    if (nm == "indices" || nm == "rowidx") {
      CHECK(count == int64_t(g.idx.size()), "%s: %s length", tag, name);
      for (int64_t i = 0; i < count; ++i)
        if (data[i] < 0 || data[i] >= g.n()) {
          CHECK(false, "%s: %s[%lld] out of range", tag, name, (long long)i);
          break;
        }
    }
  }
  CHECK(touched > 0 || g.n() == 0, "%s: no array data", tag);
  if (sum == 0x7fffffffffffLL) std::printf("%lld\n", (long long)sum);  // keep the reads live
  graph_attn_plan_destroy(p);
}

static void expect_error(const int32_t* ptr, const int32_t* idx, int64_t n, int64_t e,
                         const ga_plan_opts* o, const char* tag) {
  ga_plan* p = reinterpret_cast<ga_plan*>(0x1);
  const ga_status st = graph_attn_plan_create(ptr, idx, n, e, o, &p);
  CHECK(st != GA_OK, "%s: accepted", tag);
  if (st == GA_OK) graph_attn_plan_destroy(p);
}

int main() {
  CHECK(graph_attn_version() != nullptr, "version");
  for (int s = 0; s < 16; ++s) CHECK(graph_attn_status_string(ga_status(s)) != nullptr, "status");
  ga_plan_opts def;
  CHECK(graph_attn_plan_opts_default(&def) == GA_OK, "opts default");

  std::vector<ga_plan_opts> opts;
  opts.push_back(def);
  ga_plan_opts o = def;
  o.light_max_deg = 4; o.hub_min_deg_exclusive = 9; o.hub_chunk = 3; opts.push_back(o);
  o = def; o.light_max_deg = 0; o.hub_min_deg_exclusive = 0; o.hub_chunk = 1; opts.push_back(o);
  o = def; o.xcd_split_min_deg_exclusive = 16; o.col_xcd_split_min_deg_exclusive = 24; opts.push_back(o);
  o = def; o.light_max_deg = 1; o.xcd_split_min_deg_exclusive = 1; o.col_xcd_split_min_deg_exclusive = 1;
  o.hub_chunk = 2; o.col_hub_chunk = 3; opts.push_back(o);
  o = def; o.build_csc = 0; o.xcd_split_min_deg_exclusive = 16; opts.push_back(o);
  for (int fs : {1, 2, 4, 8}) { o = def; o.feature_slices = fs; opts.push_back(o); }
  o = def; o.light_max_deg = 4; o.col_hub_min_deg_exclusive = 5; o.col_hub_chunk = 7; opts.push_back(o);

  std::mt19937_64 rng(20261203);
  const int64_t sizes[] = {1, 2, 7, 64, 257, 3000};
  int graphs = 0;
  for (int64_t n : sizes)
    for (int sorted = 0; sorted < 2; ++sorted) {
      const Csr g = random_graph(rng, n, n > 100 ? 3 : 1, n > 100 ? 5000 : 40, sorted);
      for (size_t k = 0; k < opts.size(); ++k) {
        char tag[96];
        std::snprintf(tag, sizeof tag, "n=%lld sorted=%d opts#%zu", (long long)n, sorted, k);
        exercise(g, opts[k], tag);
      }
      ++graphs;
    }

  // degenerate graphs
  Csr empty;  // no nodes
  empty.ptr = {0};
  for (auto& op : opts) exercise(empty, op, "no nodes");
  Csr isolated;  // nodes, no edges
  isolated.ptr.assign(50, 0);
  for (auto& op : opts) exercise(isolated, op, "no edges");
  Csr star;  // one row of 100,000 edges, the rest empty; all edges from node 3
  star.ptr.assign(11, 100000);
  star.ptr[0] = 0;
  star.idx.assign(100000, 3);
  for (auto& op : opts) exercise(star, op, "star");

  // invalid CSR: arrays of the declared sizes with invalid contents, and bad sizes
  const int32_t ok_ptr[] = {0, 2, 3, 5}, ok_idx[] = {0, 1, 2, 1, 0};
  const int32_t bad_start[] = {1, 2, 3, 5};
  const int32_t bad_order[] = {0, 3, 2, 5};
  const int32_t bad_end[] = {0, 2, 3, 4};
  const int32_t big_idx[] = {0, 1, 3, 1, 0}, neg_idx[] = {0, 1, -1, 1, 0};
  expect_error(bad_start, ok_idx, 3, 5, &def, "indptr[0] != 0");
  expect_error(bad_order, ok_idx, 3, 5, &def, "indptr decreasing");
  expect_error(bad_end, ok_idx, 3, 5, &def, "indptr[n] != e");
  expect_error(ok_ptr, big_idx, 3, 5, &def, "index >= n");
  expect_error(ok_ptr, neg_idx, 3, 5, &def, "negative index");
  expect_error(ok_ptr, ok_idx, -1, 5, &def, "negative n");
  expect_error(ok_ptr, ok_idx, 3, -5, &def, "negative e");
  expect_error(nullptr, ok_idx, 3, 5, &def, "null indptr");
  expect_error(ok_ptr, nullptr, 3, 5, &def, "null indices");
  o = def; o.hub_chunk = 0; expect_error(ok_ptr, ok_idx, 3, 5, &o, "hub_chunk 0");
  o = def; o.feature_slices = 3; expect_error(ok_ptr, ok_idx, 3, 5, &o, "3 feature slices");
  o = def; o.light_max_deg = -2; expect_error(ok_ptr, ok_idx, 3, 5, &o, "negative light threshold");
  o = def; o.xcd_split_min_deg_exclusive = 8; expect_error(ok_ptr, ok_idx, 3, 5, &o, "split below light");
  ga_plan* p = nullptr;
  CHECK(graph_attn_plan_create(ok_ptr, ok_idx, 3, 5, &def, nullptr) != GA_OK, "null out");
  CHECK(graph_attn_plan_create(ok_ptr, ok_idx, 3, 5, nullptr, &p) == GA_OK, "null opts = defaults");
  if (p) graph_attn_plan_destroy(p);
  graph_attn_plan_destroy(nullptr);

  std::printf("graphs %d, option sets %zu, failures %d\n", graphs, opts.size(), failures);
  return failures ? 1 : 0;
}
