// C-ABI layer: argument validation, plan lifetime and upload, workspace sizing, kernel
// dispatch and kernel timers. Every check that can fail does so before the first HIP
// call, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "ga_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Gathers from tables of n rows of row_bytes: through buffer descriptors unless the table
// passes 4 GiB, or GRAPH_ATTN_WIDE_LOADS=1 asks for the 64-bit path everywhere.
int wide_loads(int64_t n, int64_t row_bytes) {
  const char* e = std::getenv("GRAPH_ATTN_WIDE_LOADS");
  return ga::rows_wide(n, row_bytes) || (e && e[0] == '1' && e[1] == 0);
}

// ---------------------------------------------------------------- timers
struct TimerRec {
  const char* name;
  hipEvent_t begin, end;
};

std::mutex g_timer_mu;
bool g_timer_on = false;
std::vector<TimerRec> g_recs;
std::vector<hipEvent_t> g_pool;
struct Agg {
  const char* name;
  int64_t launches;
  double ms;
};
std::vector<Agg> g_agg;

hipEvent_t pool_get() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void timer_hook(const char* name, void* stream, int begin) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  hipEvent_t e = pool_get();
  if (!e) return;
  if (hipEventRecord(e, static_cast<hipStream_t>(stream)) != hipSuccess) {
    g_pool.push_back(e);  // timers are best effort: this launch goes untimed
    return;
  }
  if (begin) {
    g_recs.push_back(TimerRec{name, e, nullptr});
  } else {
    for (auto it = g_recs.rbegin(); it != g_recs.rend(); ++it)
      if (it->end == nullptr && std::strcmp(it->name, name) == 0) {
        it->end = e;
        return;
      }
    g_pool.push_back(e);
  }
}

ga::TimerHook active_hook() {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  return g_timer_on ? timer_hook : nullptr;
}

// ---------------------------------------------------------------- plan arrays
struct ArrayRef {
  const char* name;
  const std::vector<int32_t>* (*get)(const ga_plan*);
  bool csc;
};

#define GA_REF(NAME, EXPR, CSC) \
  {NAME, [](const ga_plan* p) -> const std::vector<int32_t>* { return &(EXPR); }, CSC}
const ArrayRef kArrays[] = {
    GA_REF("indptr", p->indptr, false),
    GA_REF("indices", p->indices, false),
    GA_REF("row_light", p->rows.light, false),
    GA_REF("row_medium", p->rows.medium, false),
    GA_REF("row_hub", p->rows.hub, false),
    GA_REF("row_chunk_row", p->rows.chunk_row, false),
    GA_REF("row_chunk_begin", p->rows.chunk_begin, false),
    GA_REF("row_chunk_end", p->rows.chunk_end, false),
    GA_REF("row_hub_chunk_ptr", p->rows.hub_chunk_ptr, false),
    GA_REF("colptr", p->colptr, true),
    GA_REF("rowidx", p->rowidx, true),
    GA_REF("col_light", p->cols.light, true),
    GA_REF("col_medium", p->cols.medium, true),
    GA_REF("col_hub", p->cols.hub, true),
    GA_REF("col_chunk_row", p->cols.chunk_row, true),
    GA_REF("col_chunk_begin", p->cols.chunk_begin, true),
    GA_REF("col_chunk_end", p->cols.chunk_end, true),
    GA_REF("col_hub_chunk_ptr", p->cols.hub_chunk_ptr, true),
    GA_REF("csc_rel", p->csc_rel, true),
    GA_REF("row_sched", p->rows.sched, false),
    GA_REF("col_sched", p->cols.sched, true),
};
#undef GA_REF
constexpr int kNumArrays = sizeof(kArrays) / sizeof(kArrays[0]);

size_t device_layout(const ga_plan* p, std::vector<size_t>* offsets) {
  size_t off = 0;
  for (int i = 0; i < kNumArrays; ++i) {
    const bool present = !kArrays[i].csc || p->has_csc;
    const size_t n = present ? kArrays[i].get(p)->size() : 0;
    if (offsets) offsets->push_back(off);
    off += align_up(n * sizeof(int32_t));
  }
  return off;
}

// ---------------------------------------------------------------- argument checks
ga_status make_geometry(ga_dtype dt, int32_t heads, int32_t dim, ga::Geometry* g) {
  if (dt != GA_F32 && dt != GA_BF16) return GA_ERR_INVALID_ARG;
  if (heads < 1 || dim < 1) return GA_ERR_INVALID_ARG;
  const int64_t eb = dt == GA_F32 ? 4 : 2;
  const int64_t head_bytes = dim * eb, row_bytes = head_bytes * heads;
  if (head_bytes % 16 || row_bytes > 1024 || row_bytes % 16) return GA_ERR_UNSUPPORTED;
  g->heads = heads;
  g->dim = dim;
  g->elem_bytes = static_cast<int>(eb);
  g->G = static_cast<int>(row_bytes / 16);
  g->LH = static_cast<int>(head_bytes / 16);
  return GA_OK;
}

ga_status check_ptr(const void* p, size_t align) {
  if (!p) return GA_ERR_INVALID_ARG;
  return aligned(p, align) ? GA_OK : GA_ERR_INVALID_ARG;
}

size_t fwd_ws_bytes(const ga_plan* p, const ga::Geometry& g) {
  const size_t nc = p->rows.chunk_row.size();
  if (nc == 0) return 0;
  return align_up(nc * g.heads * 2 * sizeof(float)) +
         align_up(nc * size_t(g.heads) * g.dim * sizeof(float));
}

size_t bwd_ws_bytes(const ga_plan* p, const ga::Geometry& g) {
  const size_t F = size_t(g.heads) * g.dim;
  return align_up(size_t(p->n) * g.heads * 2 * sizeof(float)) +
         align_up(p->rows.chunk_row.size() * ga::dq_partial_floats(g.heads, g.dim) *
                  sizeof(float)) +
         align_up(p->cols.chunk_row.size() * 2 * F * sizeof(float));
}

// GATv2 backward workspace sections (bytes, each 256-aligned): record, row-chunk partials,
// column-chunk partials, da partial slots, the two fp64 buffers of the da reduction tree.
struct Gv2Layout {
  size_t ld, rows, cols, da, da64, total;
};

Gv2Layout gatv2_layout(const ga_plan* p, const ga::Geometry& g) {
  const size_t F = size_t(g.heads) * g.dim;
  Gv2Layout L;
  L.ld = align_up(size_t(p->n) * g.heads * 2 * sizeof(float));
  L.rows = align_up(p->rows.chunk_row.size() *
                    size_t(ga::gatv2_row_partial_floats(g.heads, g.dim)) * sizeof(float));
  L.cols = align_up(p->cols.chunk_row.size() * 2 * F * sizeof(float));
  const int64_t slots = ga::gatv2_da_slots(p, g);
  L.da = align_up(size_t(slots) * F * sizeof(float));
  L.da64 = align_up(size_t(ga::gatv2_reduce_rows(slots)) * F * sizeof(double));
  L.total = L.ld + L.rows + L.cols + L.da + L.da64;
  return L;
}

// Reduction geometry: F elements of `dt` are G = F*size/16 lanes (4..64, a power of two).
ga_status reduce_geometry(ga_dtype dt, int32_t features, int* G) {
  if (dt != GA_F32 && dt != GA_BF16) return GA_ERR_INVALID_ARG;
  if (features < 1) return GA_ERR_INVALID_ARG;
  const int64_t row_bytes = int64_t(features) * (dt == GA_F32 ? 4 : 2);
  if (row_bytes % 16 || row_bytes > 1024) return GA_ERR_UNSUPPORTED;
  *G = static_cast<int>(row_bytes / 16);
  return ga::reduce_supported(dt, *G) ? GA_OK : GA_ERR_UNSUPPORTED;
}

size_t reduce_fwd_ws_bytes(const ga_plan* p, int32_t features) {
  return 3 * align_up(p->rows.chunk_row.size() * size_t(features) * 4);
}

size_t reduce_bwd_ws_bytes(const ga_plan* p, int32_t features) {
  return align_up(p->cols.chunk_row.size() * size_t(features) * 4);
}

ga_status check_device(const ga_plan* p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GA_ERR_HIP;
  return dev == p->device ? GA_OK : GA_ERR_INVALID_ARG;
}

}  // namespace

namespace ga {

ga_status plan_device_check(const ga_plan* p) { return check_device(p); }

ga_status fwd_check(const ga_plan* p, ga_score score, ga_dtype dtype, int32_t heads, int32_t dim,
                    const void* a, const void* b, const void* v, const void* out,
                    const float* lse, size_t* need) {
  if (!p) return GA_ERR_INVALID_ARG;
  if (score != GA_SCORE_DOT && score != GA_SCORE_GAT) return GA_ERR_INVALID_ARG;
  ga::Geometry g;
  ga_status s = make_geometry(dtype, heads, dim, &g);
  if (s != GA_OK) return s;
  if (!ga::fwd_supported(dtype, score, g)) return GA_ERR_UNSUPPORTED;
  if (p->n > 0) {
    const size_t score_align = score == GA_SCORE_DOT ? 16 : 4;
    if ((s = check_ptr(a, score_align)) != GA_OK || (s = check_ptr(b, score_align)) != GA_OK ||
        (s = check_ptr(v, 16)) != GA_OK || (s = check_ptr(out, 16)) != GA_OK ||
        (s = check_ptr(lse, 4)) != GA_OK)
      return s;
  }
  *need = fwd_ws_bytes(p, g);
  return GA_OK;
}

ga_status fwd_enqueue(const ga_plan* p, ga_score score, ga_dtype dtype, int32_t heads,
                      int32_t dim, float scale, float neg_slope, const void* a, const void* b,
                      const void* v, void* out, float* lse, void* ws, void* stream) {
  ga_status s = check_device(p);
  if (s != GA_OK) return s;
  ga::Geometry g;
  if ((s = make_geometry(dtype, heads, dim, &g)) != GA_OK) return s;
  ga::FwdArgs args{};
  args.indptr = p->d_indptr;
  args.indices = p->d_indices;
  args.bins = p->d_rows;
  args.a = a;
  args.b = b;
  args.v = v;
  args.out = out;
  args.lse = lse;
  const size_t nc = p->rows.chunk_row.size();
  args.ws_ml = static_cast<float*>(ws);
  args.ws_acc = nc ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                              align_up(nc * heads * 2 * sizeof(float)))
                   : nullptr;
  args.sc2 = scale * 1.4426950408889634f;
  args.neg_slope = neg_slope;
  args.ld = g.G;
  args.hf = g.heads;
  args.n = static_cast<int>(p->n);
  args.wide = wide_loads(p->n, int64_t(args.ld) * 16);
  // GAT-style scores gather t_j per head, a partial line per slice: not sliced; nor are
  // plans whose chunk slots are scheduled to XCDs
  args.slices = score == GA_SCORE_DOT && p->rows.sched.empty()
                    ? ga::feature_slices(g.G, g.LH, p->opts.feature_slices,
                                         ga::kAutoSliceLanesTwoRows)
                    : 1;
  const int rc = ga::launch_fwd(dtype, score == GA_SCORE_DOT ? ga::kModeDot : ga::kModeGat, g,
                                args, p->n, stream, active_hook());
  return rc == 0 ? GA_OK : (rc < 0 ? GA_ERR_UNSUPPORTED : GA_ERR_HIP);
}

}  // namespace ga

extern "C" {

const char* graph_attn_version(void) { return "graph_attn 0.1 gfx950"; }

const char* graph_attn_status_string(ga_status s) {
  switch (s) {
    case GA_OK: return "GA_OK";
    case GA_ERR_INVALID_ARG: return "GA_ERR_INVALID_ARG: invalid argument";
    case GA_ERR_BAD_GRAPH: return "GA_ERR_BAD_GRAPH: CSR failed validation";
    case GA_ERR_UNSUPPORTED: return "GA_ERR_UNSUPPORTED: unsupported geometry or mode";
    case GA_ERR_WORKSPACE: return "GA_ERR_WORKSPACE: workspace missing or too small";
    case GA_ERR_NOT_READY: return "GA_ERR_NOT_READY: plan not uploaded or transpose missing";
    case GA_ERR_HIP: return "GA_ERR_HIP: HIP runtime error";
    case GA_ERR_HOST_ALLOC: return "GA_ERR_HOST_ALLOC: host allocation failed";
    case GA_ERR_TOO_LARGE:
      return "GA_ERR_TOO_LARGE: the call needs more than the library's fixed scratch";
  }
  return "unknown ga_status";
}

ga_status graph_attn_plan_opts_default(ga_plan_opts* o) {
  if (!o) return GA_ERR_INVALID_ARG;
  o->light_max_deg = 16;
  o->hub_min_deg_exclusive = -1;  // automatic, from the graph's size
  o->hub_chunk = -1;
  o->build_csc = 1;
  o->feature_slices = 0;
  o->col_hub_min_deg_exclusive = -1;
  o->col_hub_chunk = -1;
  o->xcd_split_min_deg_exclusive = 0;  // off
  o->col_xcd_split_min_deg_exclusive = 0;
  return GA_OK;
}

ga_status graph_attn_plan_create(const int32_t* indptr, const int32_t* indices, int64_t n,
                                 int64_t e, const ga_plan_opts* opts, ga_plan** out) {
  if (!out) return GA_ERR_INVALID_ARG;
  *out = nullptr;
  ga_plan_opts o;
  if (opts)
    o = *opts;
  else
    graph_attn_plan_opts_default(&o);
  ga_plan* p = new (std::nothrow) ga_plan();
  if (!p) return GA_ERR_HOST_ALLOC;
  const ga_status s = ga::build_plan(indptr, indices, n, e, o, p);
  if (s != GA_OK) {
    delete p;
    return s;
  }
  *out = p;
  return GA_OK;
}

ga_status graph_attn_plan_get_info(const ga_plan* p, ga_plan_info* info) {
  if (!p || !info) return GA_ERR_INVALID_ARG;
  info->n_nodes = p->n;
  info->n_edges = p->e;
  info->n_row_light = static_cast<int64_t>(p->rows.light.size());
  info->n_row_medium = static_cast<int64_t>(p->rows.medium.size());
  info->n_row_hub = static_cast<int64_t>(p->rows.hub.size());
  info->n_row_chunks = static_cast<int64_t>(p->rows.chunk_row.size());
  info->has_csc = p->has_csc;
  info->n_col_light = static_cast<int64_t>(p->cols.light.size());
  info->n_col_medium = static_cast<int64_t>(p->cols.medium.size());
  info->n_col_hub = static_cast<int64_t>(p->cols.hub.size());
  info->n_col_chunks = static_cast<int64_t>(p->cols.chunk_row.size());
  info->max_in_degree = p->max_in;
  info->max_out_degree = p->max_out;
  info->light_max_deg = p->opts.light_max_deg;
  info->hub_min_deg_exclusive = p->opts.hub_min_deg_exclusive;
  info->hub_chunk = p->opts.hub_chunk;
  info->device_bytes = static_cast<int64_t>(device_layout(p, nullptr));
  info->rows_sorted = p->rows_sorted ? 1 : 0;
  info->feature_slices = p->opts.feature_slices;
  info->col_hub_min_deg_exclusive = p->opts.col_hub_min_deg_exclusive;
  info->col_hub_chunk = p->opts.col_hub_chunk;
  info->xcd_split_min_deg_exclusive = p->opts.xcd_split_min_deg_exclusive;
  info->col_xcd_split_min_deg_exclusive = p->opts.col_xcd_split_min_deg_exclusive;
  info->n_row_sched = static_cast<int64_t>(p->rows.sched.size());
  info->n_col_sched = static_cast<int64_t>(p->cols.sched.size());
  info->uploaded = p->uploaded;
  return GA_OK;
}

ga_status graph_attn_plan_device_bytes(const ga_plan* p, size_t* bytes) {
  if (!p || !bytes) return GA_ERR_INVALID_ARG;
  *bytes = device_layout(p, nullptr);
  return GA_OK;
}

ga_status graph_attn_plan_upload(ga_plan* p, void* dev_buf, size_t bytes, void* stream) {
  if (!p) return GA_ERR_INVALID_ARG;
  std::vector<size_t> off;
  const size_t need = device_layout(p, &off);
  if (need > 0 && (!dev_buf || !aligned(dev_buf, kAlign))) return GA_ERR_INVALID_ARG;
  if (bytes < need) return GA_ERR_INVALID_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GA_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(dev_buf);
  const int32_t* ptrs[kNumArrays];
  for (int i = 0; i < kNumArrays; ++i) {
    ptrs[i] = reinterpret_cast<const int32_t*>(base + off[i]);
    const bool present = !kArrays[i].csc || p->has_csc;
    if (!present) continue;
    const std::vector<int32_t>& v = *kArrays[i].get(p);
    if (v.empty()) continue;
    if (hipMemcpyAsync(base + off[i], v.data(), v.size() * sizeof(int32_t), hipMemcpyHostToDevice,
                       s) != hipSuccess)
      return GA_ERR_HIP;
  }
  if (hipStreamSynchronize(s) != hipSuccess) return GA_ERR_HIP;
  auto bins = [&](int first, int sched, const ga::Bins& b) {
    ga::DevBins d;
    d.light = ptrs[first];
    d.medium = ptrs[first + 1];
    d.hub = ptrs[first + 2];
    d.chunk_row = ptrs[first + 3];
    d.chunk_begin = ptrs[first + 4];
    d.chunk_end = ptrs[first + 5];
    d.hub_chunk_ptr = ptrs[first + 6];
    d.n_light = static_cast<int32_t>(b.light.size());
    d.n_medium = static_cast<int32_t>(b.medium.size());
    d.n_hub = static_cast<int32_t>(b.hub.size());
    d.n_chunks = static_cast<int32_t>(b.chunk_row.size());
    d.sched = b.sched.empty() ? nullptr : ptrs[sched];
    d.n_sched = static_cast<int32_t>(b.sched.empty() ? b.chunk_row.size() : b.sched.size());
    return d;
  };
  p->d_indptr = ptrs[0];
  p->d_indices = ptrs[1];
  p->d_rows = bins(2, 19, p->rows);
  p->d_colptr = ptrs[9];
  p->d_rowidx = ptrs[10];
  p->d_cols = p->has_csc ? bins(11, 20, p->cols) : ga::DevBins{};
  p->d_csc_rel = ptrs[18];
  p->device = dev;
  p->uploaded = true;
  return GA_OK;
}

int32_t graph_attn_plan_array_count(void) { return kNumArrays; }

const char* graph_attn_plan_array_name(int32_t i) {
  return (i >= 0 && i < kNumArrays) ? kArrays[i].name : nullptr;
}

ga_status graph_attn_plan_array(const ga_plan* p, const char* name, const int32_t** data,
                                int64_t* count) {
  if (!p || !name || !data || !count) return GA_ERR_INVALID_ARG;
  for (int i = 0; i < kNumArrays; ++i) {
    if (std::strcmp(name, kArrays[i].name) != 0) continue;
    if (kArrays[i].csc && !p->has_csc) return GA_ERR_NOT_READY;
    const std::vector<int32_t>* v = kArrays[i].get(p);
    *data = v->empty() ? nullptr : v->data();
    *count = static_cast<int64_t>(v->size());
    return GA_OK;
  }
  return GA_ERR_INVALID_ARG;
}

void graph_attn_plan_destroy(ga_plan* p) { delete p; }

ga_status graph_attn_fwd_workspace_bytes(const ga_plan* p, int32_t heads, int32_t dim,
                                         size_t* bytes) {
  if (!p || !bytes || heads < 1 || dim < 1) return GA_ERR_INVALID_ARG;
  ga::Geometry g;
  g.heads = heads;
  g.dim = dim;
  *bytes = fwd_ws_bytes(p, g);
  return GA_OK;
}

ga_status graph_attn_bwd_workspace_bytes(const ga_plan* p, int32_t heads, int32_t dim,
                                         size_t* bytes) {
  if (!p || !bytes || heads < 1 || dim < 1) return GA_ERR_INVALID_ARG;
  ga::Geometry g;
  g.heads = heads;
  g.dim = dim;
  *bytes = bwd_ws_bytes(p, g);
  return GA_OK;
}

ga_status graph_attn_fwd(const ga_plan* p, ga_score score, ga_dtype dtype, int32_t heads,
                         int32_t dim, float scale, float neg_slope, const void* a, const void* b,
                         const void* v, void* out, float* lse, void* ws, size_t ws_bytes,
                         void* stream) {
  size_t need = 0;
  ga_status s = ga::fwd_check(p, score, dtype, heads, dim, a, b, v, out, lse, &need);
  if (s != GA_OK) return s;
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 16))) return GA_ERR_WORKSPACE;
  if (!p->uploaded) return GA_ERR_NOT_READY;
  if (p->n == 0) return GA_OK;
  return ga::fwd_enqueue(p, score, dtype, heads, dim, scale, neg_slope, a, b, v, out, lse, ws,
                         stream);
}

ga_status graph_attn_fwd_gatv2(const ga_plan* p, ga_dtype dtype, int32_t heads, int32_t dim,
                               float scale, float neg_slope, const void* xd, const void* xs,
                               const float* attn, void* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream) {
  if (!p) return GA_ERR_INVALID_ARG;
  ga::Geometry g;
  ga_status s = make_geometry(dtype, heads, dim, &g);
  if (s != GA_OK) return s;
  if (!ga::fwd_supported(dtype, GA_SCORE_DOT, g)) return GA_ERR_UNSUPPORTED;
  if ((s = check_ptr(attn, 16)) != GA_OK) return s;
  if (p->n > 0) {
    if ((s = check_ptr(xd, 16)) != GA_OK || (s = check_ptr(xs, 16)) != GA_OK ||
        (s = check_ptr(out, 16)) != GA_OK || (s = check_ptr(lse, 4)) != GA_OK)
      return s;
  }
  const size_t need = fwd_ws_bytes(p, g);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 16))) return GA_ERR_WORKSPACE;
  if (!p->uploaded) return GA_ERR_NOT_READY;
  if (p->n == 0) return GA_OK;
  if ((s = check_device(p)) != GA_OK) return s;
  ga::FwdArgs args{};
  args.indptr = p->d_indptr;
  args.indices = p->d_indices;
  args.bins = p->d_rows;
  args.a = xd;
  args.b = xs;
  args.v = xs;
  args.attn = attn;
  args.out = out;
  args.lse = lse;
  const size_t nc = p->rows.chunk_row.size();
  args.ws_ml = static_cast<float*>(ws);
  args.ws_acc = nc ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                              align_up(nc * heads * 2 * sizeof(float)))
                   : nullptr;
  args.sc2 = scale * 1.4426950408889634f;
  args.neg_slope = neg_slope;
  args.ld = g.G;
  args.hf = g.heads;
  args.n = static_cast<int>(p->n);
  args.wide = wide_loads(p->n, int64_t(args.ld) * 16);
  args.slices = p->rows.sched.empty()
                    ? ga::feature_slices(g.G, g.LH, p->opts.feature_slices, 0)
                    : 1;
  const int rc = ga::launch_fwd(dtype, ga::kModeGatV2, g, args, p->n, stream, active_hook());
  return rc == 0 ? GA_OK : (rc < 0 ? GA_ERR_UNSUPPORTED : GA_ERR_HIP);
}

ga_status graph_attn_bwd(const ga_plan* p, ga_score score, ga_dtype dtype, int32_t heads,
                         int32_t dim, float scale, float neg_slope, const void* q, const void* k,
                         const void* v, const void* dout, const float* lse, void* dq, void* dk,
                         void* dv, void* ws, size_t ws_bytes, void* stream) {
  if (!p) return GA_ERR_INVALID_ARG;
  if (score != GA_SCORE_DOT && score != GA_SCORE_GAT) return GA_ERR_INVALID_ARG;
  ga::Geometry g;
  ga_status s = make_geometry(dtype, heads, dim, &g);
  if (s != GA_OK) return s;
  if (!ga::bwd_supported(dtype, g)) return GA_ERR_UNSUPPORTED;
  if (p->n > 0) {
    // dot: q, k, dq, dk are [N,H,d] feature rows; gat: s, t, ds, dt are fp32 [N,H]
    const size_t qk_align = score == GA_SCORE_DOT ? 16 : 4;
    const void* f16[] = {v, dout, dv};
    const void* fqk[] = {q, k, dq, dk};
    for (const void* x : f16)
      if ((s = check_ptr(x, 16)) != GA_OK) return s;
    for (const void* x : fqk)
      if ((s = check_ptr(x, qk_align)) != GA_OK) return s;
    if ((s = check_ptr(lse, 4)) != GA_OK) return s;
  }
  if (!p->has_csc) return GA_ERR_NOT_READY;
  const size_t need = bwd_ws_bytes(p, g);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 16))) return GA_ERR_WORKSPACE;
  if (!p->uploaded) return GA_ERR_NOT_READY;
  if (p->n == 0) return GA_OK;
  if ((s = check_device(p)) != GA_OK) return s;

  ga::BwdArgs args{};
  args.indptr = p->d_indptr;
  args.indices = p->d_indices;
  args.colptr = p->d_colptr;
  args.rowidx = p->d_rowidx;
  args.rows = p->d_rows;
  args.cols = p->d_cols;
  args.q = q;
  args.k = k;
  args.v = v;
  args.dout = dout;
  args.lse = lse;
  args.dq = dq;
  args.dk = dk;
  args.dv = dv;
  char* w = static_cast<char*>(ws);
  args.ws_ld = reinterpret_cast<float*>(w);
  w += align_up(size_t(p->n) * heads * 2 * sizeof(float));
  args.ws_dq = reinterpret_cast<float*>(w);
  w += align_up(p->rows.chunk_row.size() * ga::dq_partial_floats(heads, dim) * sizeof(float));
  args.ws_dkv = reinterpret_cast<float*>(w);
  args.scale = scale;
  args.sc2 = scale * 1.4426950408889634f;
  args.neg_slope = neg_slope;
  args.ld = g.G;
  args.n = static_cast<int>(p->n);
  args.wide = wide_loads(p->n, int64_t(args.ld) * 16);
  args.hf = g.heads;
  args.slices = p->rows.sched.empty()
                    ? ga::feature_slices(g.G, g.LH, p->opts.feature_slices,
                                         ga::kAutoSliceLanesTwoRows)
                    : 1;
  args.dq_stride = static_cast<int>(ga::dq_partial_floats(heads, dim));
  const int rc = score == GA_SCORE_DOT ? ga::launch_bwd(dtype, g, args, p->n, stream, active_hook())
                                       : ga::launch_bwd_gat(dtype, g, args, stream, active_hook());
  return rc == 0 ? GA_OK : (rc < 0 ? GA_ERR_UNSUPPORTED : GA_ERR_HIP);
}

ga_status graph_attn_bwd_gatv2_workspace_bytes(const ga_plan* p, ga_dtype dtype, int32_t heads,
                                               int32_t dim, size_t* bytes) {
  if (!p || !bytes) return GA_ERR_INVALID_ARG;
  ga::Geometry g;
  const ga_status s = make_geometry(dtype, heads, dim, &g);
  if (s != GA_OK) return s;
  *bytes = gatv2_layout(p, g).total;
  return GA_OK;
}

ga_status graph_attn_bwd_gatv2(const ga_plan* p, ga_dtype dtype, int32_t heads, int32_t dim,
                               float scale, float neg_slope, const void* xd, const void* xs,
                               const float* attn, const void* dout, const float* lse, void* dxd,
                               void* dxs, float* dattn, void* ws, size_t ws_bytes,
                               void* stream) {
  if (!p) return GA_ERR_INVALID_ARG;
  ga::Geometry g;
  ga_status s = make_geometry(dtype, heads, dim, &g);
  if (s != GA_OK) return s;
  if (!ga::bwd_supported(dtype, g)) return GA_ERR_UNSUPPORTED;
  if ((s = check_ptr(attn, 16)) != GA_OK || (s = check_ptr(dattn, 16)) != GA_OK) return s;
  if (p->n > 0) {
    const void* f16[] = {xd, xs, dout, dxd, dxs};
    for (const void* x : f16)
      if ((s = check_ptr(x, 16)) != GA_OK) return s;
    if ((s = check_ptr(lse, 4)) != GA_OK) return s;
  }
  if (!p->has_csc) return GA_ERR_NOT_READY;
  const Gv2Layout L = gatv2_layout(p, g);
  if (L.total > 0 && (!ws || ws_bytes < L.total || !aligned(ws, 16))) return GA_ERR_WORKSPACE;
  if (!p->uploaded) return GA_ERR_NOT_READY;
  if ((s = check_device(p)) != GA_OK) return s;
  // an empty graph still launches the final reduction stage, which writes dattn = 0
  ga::BwdArgs args{};
  args.indptr = p->d_indptr;
  args.indices = p->d_indices;
  args.colptr = p->d_colptr;
  args.rowidx = p->d_rowidx;
  args.rows = p->d_rows;
  args.cols = p->d_cols;
  args.q = xd;
  args.k = xs;
  args.v = xs;
  args.dout = dout;
  args.lse = lse;
  args.dq = dxd;
  args.dk = dxs;
  args.dv = nullptr;
  char* w = static_cast<char*>(ws);
  args.ws_ld = reinterpret_cast<float*>(w);
  args.ws_dq = reinterpret_cast<float*>(w + L.ld);
  args.ws_dkv = reinterpret_cast<float*>(w + L.ld + L.rows);
  args.ws_da = reinterpret_cast<float*>(w + L.ld + L.rows + L.cols);
  args.ws_da64 = reinterpret_cast<double*>(w + L.ld + L.rows + L.cols + L.da);
  args.attn = attn;
  args.dattn = dattn;
  args.scale = scale;
  args.sc2 = scale * 1.4426950408889634f;
  args.neg_slope = neg_slope;
  args.n = static_cast<int>(p->n);
  args.wide = wide_loads(p->n, int64_t(g.G) * 16);
  const int rc = ga::launch_bwd_gatv2(dtype, g, args, stream, active_hook());
  return rc == 0 ? GA_OK : (rc < 0 ? GA_ERR_UNSUPPORTED : GA_ERR_HIP);
}

ga_status graph_attn_reduce_fwd_workspace_bytes(const ga_plan* p, int32_t features,
                                                size_t* bytes) {
  if (!p || !bytes || features < 1) return GA_ERR_INVALID_ARG;
  *bytes = reduce_fwd_ws_bytes(p, features);
  return GA_OK;
}

ga_status graph_attn_reduce_bwd_workspace_bytes(const ga_plan* p, int32_t features,
                                                size_t* bytes) {
  if (!p || !bytes || features < 1) return GA_ERR_INVALID_ARG;
  *bytes = reduce_bwd_ws_bytes(p, features);
  return GA_OK;
}

ga_status graph_attn_reduce_slot_bytes(const ga_plan* p, size_t* bytes) {
  if (!p || !bytes) return GA_ERR_INVALID_ARG;
  *bytes = static_cast<size_t>(ga::reduce_slot_bytes(p->max_in));
  return GA_OK;
}

ga_status graph_attn_reduce_fwd(const ga_plan* p, ga_reduce op, ga_dtype dtype,
                                int32_t features, const void* x, void* out, int32_t* arg,
                                void* slot, void* ws, size_t ws_bytes, void* stream) {
  if (!p) return GA_ERR_INVALID_ARG;
  if (op != GA_REDUCE_MAX && op != GA_REDUCE_MIN) return GA_ERR_INVALID_ARG;
  int G = 0;
  ga_status s = reduce_geometry(dtype, features, &G);
  if (s != GA_OK) return s;
  if (p->n > 0) {
    if ((s = check_ptr(x, 16)) != GA_OK || (s = check_ptr(out, 16)) != GA_OK ||
        (s = check_ptr(arg, 16)) != GA_OK)
      return s;
    if (slot && !aligned(slot, 16)) return GA_ERR_INVALID_ARG;
  }
  const size_t need = reduce_fwd_ws_bytes(p, features);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 16))) return GA_ERR_WORKSPACE;
  if (!p->uploaded) return GA_ERR_NOT_READY;
  if (p->n == 0) return GA_OK;
  if ((s = check_device(p)) != GA_OK) return s;
  ga::RedArgs args{};
  args.indptr = p->d_indptr;
  args.indices = p->d_indices;
  args.rows = p->d_rows;
  args.x = x;
  args.out = out;
  args.arg = arg;
  args.slot = slot;
  args.slot_bytes = ga::reduce_slot_bytes(p->max_in);
  args.rows_sorted = p->rows_sorted;
  args.ld = G;
  args.n = static_cast<int>(p->n);
  args.wide = wide_loads(p->n, int64_t(args.ld) * 16);
  args.slices = p->rows.sched.empty() ? ga::feature_slices(G, 1, p->opts.feature_slices, 0) : 1;
  if (need > 0) {
    args.ws_val = static_cast<float*>(ws);
    args.ws_idx = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + need / 3);
    args.ws_pos = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + 2 * (need / 3));
  }
  const int rc = ga::launch_reduce(dtype, false, op == GA_REDUCE_MAX ? ga::kReduceMax
                                                                     : ga::kReduceMin,
                                   G, args, stream, active_hook());
  return rc == 0 ? GA_OK : (rc < 0 ? GA_ERR_UNSUPPORTED : GA_ERR_HIP);
}

ga_status graph_attn_reduce_bwd(const ga_plan* p, ga_dtype dtype, int32_t features,
                                const int32_t* arg, const void* slot, const void* dout,
                                void* dx, void* ws, size_t ws_bytes, void* stream) {
  if (!p) return GA_ERR_INVALID_ARG;
  int G = 0;
  ga_status s = reduce_geometry(dtype, features, &G);
  if (s != GA_OK) return s;
  if (p->n > 0) {
    if ((s = check_ptr(slot ? slot : static_cast<const void*>(arg), 16)) != GA_OK ||
        (s = check_ptr(dout, 16)) != GA_OK || (s = check_ptr(dx, 16)) != GA_OK)
      return s;
  }
  if (!p->has_csc) return GA_ERR_NOT_READY;
  const size_t need = reduce_bwd_ws_bytes(p, features);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 16))) return GA_ERR_WORKSPACE;
  if (!p->uploaded) return GA_ERR_NOT_READY;
  if (p->n == 0) return GA_OK;
  if ((s = check_device(p)) != GA_OK) return s;
  ga::RedArgs args{};
  args.colptr = p->d_colptr;
  args.rowidx = p->d_rowidx;
  args.cols = p->d_cols;
  args.arg_in = slot ? nullptr : arg;
  args.slot_in = slot;
  args.csc_rel = p->d_csc_rel;
  args.slot_bytes = ga::reduce_slot_bytes(p->max_in);
  args.ld = G;
  args.n = static_cast<int>(p->n);
  args.wide = wide_loads(p->n, int64_t(args.ld) * 16);
  args.slices = p->cols.sched.empty() ? ga::feature_slices(G, 1, p->opts.feature_slices, 0) : 1;
  args.dout = dout;
  args.dx = dx;
  args.ws_sum = need > 0 ? static_cast<float*>(ws) : nullptr;
  const int rc = ga::launch_reduce(dtype, true, ga::kReduceMax, G, args, stream, active_hook());
  return rc == 0 ? GA_OK : (rc < 0 ? GA_ERR_UNSUPPORTED : GA_ERR_HIP);
}

ga_status graph_attn_timer_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  g_timer_on = enable != 0;
  return GA_OK;
}

ga_status graph_attn_timer_reset(void) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  for (auto& r : g_recs) {
    if (r.begin) g_pool.push_back(r.begin);
    if (r.end) g_pool.push_back(r.end);
  }
  g_recs.clear();
  g_agg.clear();
  return GA_OK;
}

int32_t graph_attn_timer_count(void) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  g_agg.clear();
  for (const auto& r : g_recs) {
    if (!r.end) continue;
    if (hipEventSynchronize(r.end) != hipSuccess) continue;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.begin, r.end) != hipSuccess) continue;
    bool found = false;
    for (auto& a : g_agg)
      if (std::strcmp(a.name, r.name) == 0) {
        a.launches++;
        a.ms += ms;
        found = true;
        break;
      }
    if (!found) g_agg.push_back(Agg{r.name, 1, ms});
  }
  return static_cast<int32_t>(g_agg.size());
}

ga_status graph_attn_timer_read(int32_t index, const char** name, int64_t* launches,
                                double* total_ms) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  if (index < 0 || index >= static_cast<int32_t>(g_agg.size()) || !name || !launches ||
      !total_ms)
    return GA_ERR_INVALID_ARG;
  *name = g_agg[index].name;
  *launches = g_agg[index].launches;
  *total_ms = g_agg[index].ms;
  return GA_OK;
}

ga_status graph_attn_gather_probe(const ga_plan* p, ga_dtype dtype, int32_t heads, int32_t dim,
                                  const void* row_a, const void* row_b, const void* k,
                                  const void* v, void* sink, void* stream) {
  if (!p) return GA_ERR_INVALID_ARG;
  ga::Geometry g;
  ga_status s = make_geometry(dtype, heads, dim, &g);
  if (s != GA_OK) return s;
  if (g.G < 4) return GA_ERR_UNSUPPORTED;
  if (p->n > 0) {
    if ((s = check_ptr(k, 16)) != GA_OK) return s;
    for (const void* x : {row_a, row_b, v})
      if (x && !aligned(x, 16)) return GA_ERR_INVALID_ARG;
  }
  if ((s = check_ptr(sink, 16)) != GA_OK) return s;
  if (!p->uploaded) return GA_ERR_NOT_READY;
  if (p->n == 0) return GA_OK;
  if ((s = check_device(p)) != GA_OK) return s;
  ga::ProbeLaunch L{};
  L.ptr = p->d_indptr;
  L.idx = p->d_indices;
  L.bins = p->d_rows;
  L.side_a = row_a;
  L.side_b = row_b;
  L.gx = k;
  L.gy = v;
  L.sink = sink;
  L.G = g.G;
  L.LH = g.LH;
  L.heads = g.heads;
  // the forward's feature slices: automatic 256-byte slices when two rows are gathered per
  // edge, none for one row; none on a plan with an XCD schedule
  L.slices = p->rows.sched.empty()
                 ? ga::feature_slices(g.G, g.LH, p->opts.feature_slices,
                                      v ? ga::kAutoSliceLanesTwoRows : 0)
                 : 1;
  const int rc = ga::launch_gather_probe_rows(L, stream, active_hook());
  return rc == 0 ? GA_OK : (rc < 0 ? GA_ERR_UNSUPPORTED : GA_ERR_HIP);
}

ga_status graph_attn_gather_probe_cols(const ga_plan* p, ga_dtype dtype, int32_t heads,
                                       int32_t dim, const void* k, const void* v, const void* q,
                                       const void* dout, const float* record, void* sink,
                                       void* stream) {
  if (!p) return GA_ERR_INVALID_ARG;
  ga::Geometry g;
  ga_status s = make_geometry(dtype, heads, dim, &g);
  if (s != GA_OK) return s;
  if (g.G < 4) return GA_ERR_UNSUPPORTED;
  if (p->n > 0) {
    if ((s = check_ptr(dout, 16)) != GA_OK) return s;
    for (const void* x : {k, v, q})
      if (x && !aligned(x, 16)) return GA_ERR_INVALID_ARG;
    if (record && !aligned(record, 8)) return GA_ERR_INVALID_ARG;
  }
  if ((s = check_ptr(sink, 16)) != GA_OK) return s;
  if (!p->has_csc) return GA_ERR_NOT_READY;
  if (!p->uploaded) return GA_ERR_NOT_READY;
  if (p->n == 0) return GA_OK;
  if ((s = check_device(p)) != GA_OK) return s;
  ga::ProbeLaunch L{};
  L.ptr = p->d_colptr;
  L.idx = p->d_rowidx;
  L.bins = p->d_cols;
  L.side_a = k;
  L.side_b = v;
  L.gx = dout;
  L.gy = q;
  L.rec = record;
  L.sink = sink;
  L.G = g.G;
  L.LH = g.LH;
  L.heads = g.heads;
  L.slices = 1;
  const int rc = ga::launch_gather_probe_cols(L, stream, active_hook());
  return rc == 0 ? GA_OK : (rc < 0 ? GA_ERR_UNSUPPORTED : GA_ERR_HIP);
}

ga_status graph_attn_gather_probe_random(int32_t row_bytes, const void* table, int64_t table_rows,
                                         int64_t n_gathers, uint64_t seed, void* sink,
                                         void* stream) {
  if (row_bytes != 64 && row_bytes != 128 && row_bytes != 256 && row_bytes != 512 &&
      row_bytes != 1024)
    return GA_ERR_UNSUPPORTED;
  if (table_rows < 1 || table_rows > int64_t(0xffffffff) || n_gathers < 0)
    return GA_ERR_INVALID_ARG;
  ga_status s;
  if ((s = check_ptr(table, 16)) != GA_OK || (s = check_ptr(sink, 16)) != GA_OK) return s;
  if (n_gathers == 0) return GA_OK;
  const int rc = ga::launch_gather_probe_random(row_bytes / 16, table, table_rows, n_gathers,
                                                seed, sink, stream, active_hook());
  return rc == 0 ? GA_OK : (rc < 0 ? GA_ERR_UNSUPPORTED : GA_ERR_HIP);
}

ga_status graph_attn_copy_probe(void* dst, const void* src, size_t bytes, void* stream) {
  if (bytes % 16) return GA_ERR_INVALID_ARG;
  if (bytes == 0) return GA_OK;
  if (!dst || !src || !aligned(dst, 16) || !aligned(src, 16)) return GA_ERR_INVALID_ARG;
  const int rc = ga::launch_copy(dst, src, bytes, stream, active_hook());
  return rc == 0 ? GA_OK : GA_ERR_HIP;
}

}  // extern "C"
