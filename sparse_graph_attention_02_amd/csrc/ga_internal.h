// Internal declarations shared by the host planner, the C-ABI layer and the kernel
// launchers. Not part of the public interface (include/graph_attn.h is).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "graph_attn.h"

namespace ga {

// L2 partitions (XCDs) of the GPU; workgroups are dealt to them round-robin by id. Waves
// per workgroup of the kernels that run scheduled chunk slots (kWavesPerBlock on device).
constexpr int kXcds = 8;
constexpr int kWavesPerSlotBlock = 4;

// One degree-binned view of a CSR-like structure (the CSR itself, or its transpose).
struct Bins {
  std::vector<int32_t> light, medium, hub;               // ids, degree desc / id asc
  std::vector<int32_t> chunk_row, chunk_begin, chunk_end;  // hub chunks, hub by hub
  std::vector<int32_t> hub_chunk_ptr;                      // [n_hub + 1]
  std::vector<int32_t> sched;  // dispatch slot -> chunk id or -1 (empty: slot = chunk id)
};

// Device pointers of one Bins (into the caller's plan buffer).
struct DevBins {
  const int32_t* light = nullptr;
  const int32_t* medium = nullptr;
  const int32_t* hub = nullptr;
  const int32_t* chunk_row = nullptr;
  const int32_t* chunk_begin = nullptr;
  const int32_t* chunk_end = nullptr;
  const int32_t* hub_chunk_ptr = nullptr;
  const int32_t* sched = nullptr;  // null: chunk slots run in chunk order
  int32_t n_light = 0, n_medium = 0, n_hub = 0, n_chunks = 0;
  int32_t n_sched = 0;  // chunk slots: sched's length, or n_chunks without it
};

}  // namespace ga

struct ga_plan {
  int64_t n = 0, e = 0;
  ga_plan_opts opts{};
  std::vector<int32_t> indptr, indices;
  ga::Bins rows;
  bool has_csc = false;
  std::vector<int32_t> colptr, rowidx;
  std::vector<int32_t> csc_rel;  // per transpose entry: the edge's position in its CSR row
  ga::Bins cols;
  int64_t max_in = 0, max_out = 0;
  bool rows_sorted = true;  // every row's neighbour ids are non-decreasing

  // device copy (caller-owned memory)
  bool uploaded = false;
  int device = -1;
  const int32_t* d_indptr = nullptr;
  const int32_t* d_indices = nullptr;
  const int32_t* d_colptr = nullptr;
  const int32_t* d_rowidx = nullptr;
  const int32_t* d_csc_rel = nullptr;
  ga::DevBins d_rows, d_cols;
};

namespace ga {

// Largest edge count a plan accepts: 2^31 - 2^16.
constexpr int64_t kMaxEdges = (int64_t(1) << 31) - (int64_t(1) << 16);

// Forward entry points (api.cpp), shared by graph_attn_fwd and graph_attn_fwd_noalloc.
// fwd_check runs every argument check that needs no HIP call and reports the workspace
// bytes the call needs; fwd_enqueue checks that the current device is the plan's and
// launches the forward with workspace `ws` (the plan uploaded, N > 0). plan_device_check
// is the device check alone.
ga_status fwd_check(const ga_plan* p, ga_score score, ga_dtype dtype, int32_t heads, int32_t dim,
                    const void* a, const void* b, const void* v, const void* out,
                    const float* lse, size_t* need);
ga_status fwd_enqueue(const ga_plan* p, ga_score score, ga_dtype dtype, int32_t heads,
                      int32_t dim, float scale, float neg_slope, const void* a, const void* b,
                      const void* v, void* out, float* lse, void* ws, void* stream);
ga_status plan_device_check(const ga_plan* p);

// Planner (plan.cpp). Validates and builds every host array.
ga_status build_plan(const int32_t* indptr, const int32_t* indices, int64_t n, int64_t e,
                     const ga_plan_opts& opts, ga_plan* p);

// Feature geometry shared by the launchers: a "row" is H*d elements = G lanes x 16 bytes,
// a head spans LH lanes.
struct Geometry {
  int heads = 0, dim = 0, elem_bytes = 0;
  int G = 0;   // lanes per feature row (row bytes / 16)
  int LH = 0;  // lanes per head (head bytes / 16)
};

// Feature slices for a row of G lanes with heads of LH lanes (LH = 1 when the kernel has
// no heads): S divides 8 and G and a slice holds whole heads. A requested S (2, 4 or 8)
// is lowered until it fits with slices of at least 4 lanes. requested = 0 (auto) picks the
// largest S whose slices are at least auto_lanes lanes, or 1 when auto_lanes is 0: each
// slice repeats the per-edge fixed work (index broadcast, head sums, exponentials), which
// measured slower than the L2 gain for kernels that gather one row per edge and faster
// with 256-byte slices (16 lanes) for the two-row gathers of the dot forward and dQ pass.
inline int feature_slices(int G, int LH, int requested, int auto_lanes) {
  auto fits = [&](int S, int min_lanes) {
    return G % S == 0 && (G / S) % LH == 0 && G / S >= min_lanes;
  };
  if (requested == 1) return 1;
  if (requested > 1) {
    for (int S = requested; S > 1; S /= 2)
      if (fits(S, 4)) return S;
    return 1;
  }
  int best = 1;
  if (auto_lanes > 0)
    for (int S = 2; S <= 8; S *= 2)
      if (fits(S, auto_lanes)) best = S;
  return best;
}
constexpr int kAutoSliceLanesTwoRows = 16;  // auto slices of the dot forward / dQ pass

// A buffer descriptor addresses its table with a 32-bit byte offset, so gathers read
// through one only while n rows of row_bytes fit in 4 GiB; larger tables take plain
// 64-bit loads.
inline int rows_wide(int64_t n, int64_t row_bytes) { return n * row_bytes > (int64_t(1) << 32); }

// Forward kernels (fwd.hip).
struct FwdArgs {
  const int32_t* indptr;
  const int32_t* indices;
  DevBins bins;
  const void* a;  // q (dot) or s (gat)
  const void* b;  // k (dot) or t (gat)
  const void* v;
  const float* attn;  // GATv2 attention vector [H*d] (null otherwise)
  void* out;
  float* lse;
  float* ws_ml;   // [n_chunks][H][2]  (m in log2 units, l)
  float* ws_acc;  // [n_chunks][H*d]
  float sc2;      // scale * log2(e)
  float neg_slope;
  int ld;         // feature row stride in 16-byte lanes (the full row)
  int hf;         // heads per node (stride of lse / s / t / partial (m, l))
  int slices;     // feature slices of the main kernel (1, 2, 4 or 8)
  int n;          // nodes (rows of every node-indexed tensor)
  int wide;       // gathered tables span more than one 4 GiB buffer window (rows_wide)
};

// Backward kernels (bwd.hip).
struct BwdArgs {
  const int32_t* indptr;
  const int32_t* indices;
  const int32_t* colptr;
  const int32_t* rowidx;
  DevBins rows, cols;
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* ws_ld;    // [N][H][2]: (lse * log2 e, D)
  float* ws_dq;    // [n_row_chunks][dq_partial_floats(H, d)]
  float* ws_dkv;   // [n_col_chunks][2][H*d]
  float scale;
  float sc2;       // scale * log2(e)
  float neg_slope; // LeakyReLU slope (GAT and GATv2 scores)
  int ld;            // feature row stride in 16-byte lanes (the full row)
  int hf;            // heads per node (stride of lse and of the records)
  int slices;        // feature slices of the dQ pass (1, 2, 4 or 8)
  int dq_stride;     // floats per dQ chunk partial of the full row (dq_partial_floats)
  int n;             // nodes (rows of every node-indexed tensor)
  int wide;          // gathered tables span more than one 4 GiB buffer window (rows_wide)
  // GATv2 only
  const float* attn;  // attention vector [H*d]
  float* dattn;       // its gradient [H*d]
  float* ws_da;       // da partials [n_slots][H*d]
  double* ws_da64;    // da reduction tree: two fp64 buffers of gatv2_reduce_rows() rows of H*d
};

// fp32 floats per hub-row chunk partial of the row pass: A [H*d], B [H*d], D [H], L [H]
// (D and L padded together to a multiple of 4).
inline int64_t dq_partial_floats(int64_t heads, int64_t dim) {
  return 2 * heads * dim + (2 * heads + 3) / 4 * 4;
}

// Forward score modes of the kernels (ga_score values, plus GATv2 which has its own entry
// point because it takes the attention vector).
enum FwdMode { kModeDot = 0, kModeGat = 1, kModeGatV2 = 2 };

// Returns false when the geometry/dtype/score combination has no compiled kernels.
bool fwd_supported(ga_dtype dt, ga_score sc, const Geometry& g);
bool bwd_supported(ga_dtype dt, const Geometry& g);

// Enqueue the forward / backward kernels. A non-null hook is called before (begin = 1)
// and after (begin = 0) each launch with the kernel's name (the library's event timers).
// Both return hipSuccess or the first launch error (as int to keep HIP headers out).
typedef void (*TimerHook)(const char* name, void* stream, int begin);
int launch_fwd(ga_dtype dt, int mode, const Geometry& g, const FwdArgs& a, int64_t n,
               void* stream, TimerHook hook);
int launch_bwd(ga_dtype dt, const Geometry& g, const BwdArgs& a, int64_t n, void* stream,
               TimerHook hook);
// GAT-style score: q/k/dq/dk carry s/t/ds/dt (fp32 [N, H]).
int launch_bwd_gat(ga_dtype dt, const Geometry& g, const BwdArgs& a, void* stream,
                   TimerHook hook);
// GATv2: q/k/dq/dk carry xd/xs/dxd/dxs ([N, H, d]); attn/dattn/ws_da/ws_da64 set.
int launch_bwd_gatv2(ga_dtype dt, const Geometry& g, const BwdArgs& a, void* stream,
                     TimerHook hook);
// dattn partial slots of the GATv2 backward (row waves, hub rows, column blocks, hub
// columns), the floats of one row-chunk partial, and the fp64 rows of the dattn reduction
// buffers (total, and the first buffer's share).
int64_t gatv2_da_slots(const ga_plan* p, const Geometry& g);
int64_t gatv2_row_partial_floats(int heads, int dim);  // A1 B1 [H*d], D L [H] (padded)
int64_t gatv2_reduce_rows(int64_t n_slots);
int64_t gatv2_reduce_rows_a(int64_t n_slots);
// Neighbourhood min / max reduction (reduce.hip). Rows of F elements are G lanes x 16 B.
enum ReduceOp { kReduceMax = 0, kReduceMin = 1 };
struct RedArgs {
  const int32_t* indptr;
  const int32_t* indices;
  const int32_t* colptr;
  const int32_t* rowidx;
  DevBins rows, cols;
  const int32_t* csc_rel;  // per transpose entry: the edge's position in its CSR row
  int slot_bytes;          // 2 or 4: width of the slot array
  bool rows_sorted;        // host-side: every row's neighbour ids non-decreasing
  int ld;                  // feature row stride in 16-byte lanes (the full row)
  int slices;              // feature slices of the main kernels (1, 2, 4 or 8)
  int n;                   // nodes (rows of every node-indexed tensor)
  int wide;                // gathered tables span more than one 4 GiB buffer window
  // forward
  const void* x;     // [N, F]
  void* out;         // [N, F]
  int32_t* arg;      // [N, F]
  void* slot;        // [N, F] row positions of the winners (optional)
  float* ws_val;     // hub chunk partials [n_row_chunks][F]: values,
  int32_t* ws_idx;   //                                      ids
  int32_t* ws_pos;   //                                      and edge indices
  // backward: match on slot_in when it is set, else on arg_in
  const int32_t* arg_in;  // [N, F] (the forward's arg)
  const void* slot_in;    // [N, F] (the forward's slot)
  const void* dout;       // [N, F]
  void* dx;               // [N, F]
  float* ws_sum;          // hub column partial sums [n_col_chunks][F]
};
// Width of the slot array of a plan: 2 bytes when no row has more than 65535 edges, so
// that every position (at most 65534) differs from the all-ones "no winner" slot.
inline int reduce_slot_bytes(int64_t max_in_degree) { return max_in_degree <= 65535 ? 2 : 4; }
bool reduce_supported(ga_dtype dt, int G);
int launch_reduce(ga_dtype dt, bool backward, int op, int G, const RedArgs& a, void* stream,
                  TimerHook hook);
int launch_copy(void* dst, const void* src, size_t bytes, void* stream, TimerHook hook);
// Gather-only probes (probe.hip). Rows: the forward's / dQ pass's work list over
// (ptr, idx) = (indptr, indices) with the row bins; columns: the dK/dV pass's work list over
// (colptr, rowidx) with the column bins. side_a / side_b: operand rows read once per work
// item; gx / gy: rows gathered per edge (gy may be null); rec: the columns' per-edge
// (lse, D) record [N][heads] (may be null). G lanes per feature row, LH per head; the rows
// probe runs in `slices` feature slices.
struct ProbeLaunch {
  const int32_t* ptr;
  const int32_t* idx;
  DevBins bins;
  const void* side_a;
  const void* side_b;
  const void* gx;
  const void* gy;
  const void* rec;
  void* sink;
  int G, LH, heads, slices;
};
int launch_gather_probe_rows(const ProbeLaunch& p, void* stream, TimerHook hook);
int launch_gather_probe_cols(const ProbeLaunch& p, void* stream, TimerHook hook);
// Random rows of a table of `rows` rows of G lanes, n gathers.
int launch_gather_probe_random(int G, const void* table, int64_t rows, int64_t n, uint64_t seed,
                               void* sink, void* stream, TimerHook hook);

}  // namespace ga
