/*
 * graph_attn.h -- C ABI of the fused CSR graph-attention library for AMD MI355X (gfx950),
 * with the degree-aware min / max neighbourhood reduction beside it (end of this file).
 *
 * What the library computes is the attention-based layer family of "On Efficient Scaling
 * of GNNs via IO-Aware Layers Implementations" (gist.science explainer of arXiv
 * 2605.31500), Technical Summary > Methodology: for every destination node of a CSR
 * graph, score each neighbour edge, normalise the scores with an online softmax whose
 * running statistics stay in registers, and accumulate the weighted neighbour values in
 * one streaming pass, so no edge-sized score or probability tensor is ever stored. The
 * backward keeps one log-sum-exp per node and head and recomputes the attention weights;
 * it reads a cached transpose of the adjacency (same section, SpMM paragraph: transposed
 * adjacency precomputed for the backward pass), so dK/dV need no atomics. Rows are
 * binned by degree (same section, reduction paragraph: light / heavy split by a degree
 * threshold, heavy rows reduced over edge chunks in parallel).
 *
 * Score forms (dot: Graph-Transformer layer; gat: GAT-style layer), per head h:
 *     dot:  e_ij = scale * sum_c q[i,h,c] k[j,h,c]
 *     gat:  e_ij = scale * LeakyReLU_{neg_slope}(s[i,h] + t[j,h])
 *     out[i,h,:] = sum_j softmax_j(e_ij) v[j,h,:],   lse[i,h] = ln sum_j exp(e_ij)
 * A row with no neighbours gives out = 0 and lse = -inf. The GATv2 score has entry points
 * of its own (graph_attn_fwd_gatv2, graph_attn_bwd_gatv2), as it takes an attention vector.
 *
 * Conventions shared by every call
 *   Graph: CSR with int32 indptr [N+1] and indices [E], row i = destination, indices =
 *     its sources. Parallel edges count with multiplicity. N < 2^31 and E <= 2^31 - 2^16
 *     (kernels walk edge positions in 32-bit integers); larger graphs: GA_ERR_INVALID_ARG.
 *   Features: node-major, contiguous [N, H, d] in the call's dtype (fp32 or bf16), each
 *     pointer 16-byte aligned, H*d*sizeof(dtype) a multiple of 16 bytes and at most 1024
 *     bytes, d*sizeof(dtype) a power of two between 32 and 1024 bytes dividing the row.
 *     lse is fp32 [N, H].  GAT mode: s and t are fp32 [N, H] (4-byte aligned). N is the
 *     plan's node count: calls receive pointers only and cannot check buffer sizes, so
 *     every per-node array must hold N rows (kernels index them by node id).
 *   Ownership: the caller allocates and frees every device buffer (features, outputs,
 *     the plan's device copy, workspaces). The library never calls hipMalloc/hipFree;
 *     it owns only the host-side plan metadata, and the fixed scratch array of
 *     graph_attn_fwd_noalloc (part of its device code, not an allocation).
 *   Streams: `stream` is a hipStream_t (NULL = the default stream). fwd/bwd only enqueue
 *     work and return; results are ready when the stream reaches them. They neither
 *     allocate nor synchronise nor memset, so they can be captured into a HIP graph
 *     (with the kernel timers off) and replayed.
 *   Errors: every call returns a ga_status; nothing throws or aborts across the ABI.
 *     Argument checks run before any HIP call, so an invalid call enqueues nothing.
 *   Determinism: no atomics anywhere; partial states merge in a fixed order, so two runs
 *     on the same inputs are bitwise identical.
 *   Gathers: the forward, the GATv2 row pass and the min / max forward read neighbour
 *     rows through buffer descriptors while N * row bytes <= 2^32, and with plain 64-bit
 *     loads past that (results are the same either way). Setting the environment
 *     variable GRAPH_ATTN_WIDE_LOADS=1 makes every call take the 64-bit path (read at
 *     each call; a testing aid).
 *   Non-finite inputs: a NaN or infinity in node j's features reaches only the rows
 *     that list j (and, in the backward, what those rows feed), as in the plain
 *     definition. A step folds several edges; its unused slots read zeros (a buffer
 *     record past the table, which loads nothing) or an edge of the same row, with a
 *     zero weight, never another node's row.
 */
#ifndef GRAPH_ATTN_H
#define GRAPH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GA_OK = 0,
  GA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misaligned pointer, bad enum */
  GA_ERR_BAD_GRAPH = 2,    /* CSR fails validation (indptr[0]!=0, not monotone,
                              indptr[N]!=E, index outside [0,N)) */
  GA_ERR_UNSUPPORTED = 3,  /* feature geometry or mode this build does not implement */
  GA_ERR_WORKSPACE = 4,    /* workspace pointer null or smaller than required */
  GA_ERR_NOT_READY = 5,    /* plan not uploaded, or transpose missing for backward */
  GA_ERR_HIP = 6,          /* a HIP runtime call or kernel launch failed */
  GA_ERR_HOST_ALLOC = 7,   /* host memory for the plan could not be allocated */
  GA_ERR_TOO_LARGE = 8     /* the call needs more scratch memory than the library's fixed
                              scratch holds (graph_attn_fwd_noalloc) */
} ga_status;

typedef enum { GA_F32 = 0, GA_BF16 = 1 } ga_dtype;
typedef enum { GA_SCORE_DOT = 0, GA_SCORE_GAT = 1 } ga_score;

/* Degree-binning thresholds. Rows (and, for the transpose, columns) with degree
 * <= light_max_deg are "light" (one lane group per row); degree in
 * (light_max_deg, hub_min_deg_exclusive] is "medium" (one wavefront per row); larger
 * rows are "hubs", cut into chunks of hub_chunk edges that separate wavefronts reduce,
 * merged in ascending chunk order. build_csc != 0 also builds the transpose needed by
 * graph_attn_bwd. feature_slices: the kernels that gather whole feature rows per edge
 * (the dot and GATv2 forwards, the dot backward's row pass, both reduction passes) split
 * each row into S slices of whole heads and deal the slices to the GPU's 8 L2 partitions
 * (XCDs), so each partition caches a slice of every hot row instead of whole rows. Each
 * slice repeats the per-edge fixed work, so it pays only where rows are wide: 0 =
 * automatic (the dot forward and the dot backward's row pass, which gather two rows per
 * edge, take the largest S dividing 8 whose slices are at least 256 bytes; the other
 * kernels 1), 1 = off, 2, 4 or 8 = that many slices for every kernel named above,
 * lowered until they hold whole heads of at least 64 bytes. Results agree to rounding
 * (bit for bit for the reduction, whose selection is exact).
 * col_hub_min_deg_exclusive and col_hub_chunk are the hub threshold and chunk of the
 * transpose's column bins (light columns use light_max_deg).
 * A hub threshold or chunk of -1 (the defaults) is chosen from the graph: the row hub
 * threshold is the power of two nearest E / 8192 kept within [256, 8192] (about one
 * wavefront's share of the edges when ~8192 are in flight, so no single row item becomes
 * the tail), at least light_max_deg; the row chunk max(256, threshold / 4); the column
 * threshold min(1024, row threshold) and column chunk min(512, row chunk), as the column
 * passes do more work per edge. graph_attn_plan_get_info reports the values used.
 * xcd_split_min_deg_exclusive (rows) and col_xcd_split_min_deg_exclusive (transpose
 * columns), 0 = off (the default): rows longer than this become hubs whose edges the plan
 * regroups by source id mod 8 (stable within a group, in the plan's own copy of the CSR;
 * columns: destinations by id mod 8), each group chunked separately, and the chunks are
 * scheduled so that group p runs on the XCD whose workgroups have id = p mod 8. Each XCD's
 * 4 MB L2 then holds hot rows of one eighth of the nodes instead of all of them. The
 * forward (every score), the dot backward's dQ and dK/dV passes, both GAT-style backward
 * passes, the GATv2 column pass and both min/max reduction passes run this schedule; the
 * GATv2 row pass runs the chunks in order. The scheduled passes run unsliced on a split
 * plan (feature_slices does not apply to them). Attention results agree with an unsplit
 * plan to rounding (the sum order within a row changes); the reduction's out and arg are
 * identical, and its slots are positions in the plan's rows (the exported "indices").
 * Constraints: light_max_deg >= 0; an explicit threshold >= light_max_deg; an explicit
 * chunk >= 1; feature_slices in {0, 1, 2, 4, 8}; a split threshold 0 or >= light_max_deg.
 * A plan whose work items (scheduled chunk slots, medium and light rows) would exceed
 * 2^31 - 1 is refused with GA_ERR_UNSUPPORTED. */
typedef struct {
  int32_t light_max_deg;
  int32_t hub_min_deg_exclusive;
  int32_t hub_chunk;
  int32_t build_csc;
  int32_t feature_slices;
  int32_t col_hub_min_deg_exclusive;
  int32_t col_hub_chunk;
  int32_t xcd_split_min_deg_exclusive;
  int32_t col_xcd_split_min_deg_exclusive;
} ga_plan_opts;

/* Counts describing a built plan (all int64 so the struct has no padding). */
typedef struct {
  int64_t n_nodes, n_edges;
  int64_t n_row_light, n_row_medium, n_row_hub, n_row_chunks;
  int64_t has_csc;
  int64_t n_col_light, n_col_medium, n_col_hub, n_col_chunks;
  int64_t max_in_degree, max_out_degree;
  int64_t light_max_deg, hub_min_deg_exclusive, hub_chunk;  /* as used (automatic resolved) */
  int64_t device_bytes;
  int64_t uploaded;
  int64_t rows_sorted;  /* 1 when every row's neighbour ids are non-decreasing */
  int64_t feature_slices;  /* the option as given (0 = automatic) */
  int64_t col_hub_min_deg_exclusive, col_hub_chunk;      /* as used */
  int64_t xcd_split_min_deg_exclusive, col_xcd_split_min_deg_exclusive;
  int64_t n_row_sched, n_col_sched;  /* scheduled chunk slots (0: chunk order) */
} ga_plan_info;

typedef struct ga_plan ga_plan; /* opaque; host metadata owned by the library */

/* Library version string, e.g. "graph_attn 0.1 gfx950". Never NULL. */
const char* graph_attn_version(void);

/* Human-readable name of a status code. Never NULL. */
const char* graph_attn_status_string(ga_status status);

/* Fill *opts with the defaults: light_max_deg 16, hub thresholds and chunks -1 (chosen
 * from the graph), build_csc 1, feature_slices 0 (automatic), both split thresholds 0
 * (off). */
ga_status graph_attn_plan_opts_default(ga_plan_opts* opts);

/* Build a plan from a host CSR graph (the planner of the degree-aware tiling; runs on the
 * host, O(N + E), no HIP calls). The CSR is always validated; GA_ERR_BAD_GRAPH on failure.
 * Bins: each bin lists its rows by degree descending, ties by ascending row id. Hub row
 * chunks: [indptr[i] + k*C, min(indptr[i] + (k+1)*C, indptr[i+1])), listed hub by hub;
 * a split row (see xcd_split_min_deg_exclusive) is listed by group, each group's range
 * cut the same way, and "indices" is the regrouped CSR. "row_sched" / "col_sched": the
 * chunk scheduled in each dispatch slot (-1 = none), empty when nothing is split.
 * Transpose (build_csc): colptr [N+1] and rowidx [E], destinations ascending within each
 * column (the order a stable scatter over rows produces; split columns regrouped as
 * above), and csc_rel [E], for each
 * transpose entry the position of that edge within its CSR row (k - indptr[i] for CSR
 * edge k of row i); column bins/chunks follow the same rules on out-degree.
 * indptr_host/indices_host are only read during the call (indices_host may be NULL when
 * n_edges == 0). opts NULL = defaults. On success *out receives a plan to be released
 * with graph_attn_plan_destroy. */
ga_status graph_attn_plan_create(const int32_t* indptr_host, const int32_t* indices_host,
                                 int64_t n_nodes, int64_t n_edges, const ga_plan_opts* opts,
                                 ga_plan** out);

/* Counts of a plan. */
ga_status graph_attn_plan_get_info(const ga_plan* plan, ga_plan_info* info);

/* Bytes of device memory the plan's device copy needs (the CSR, bins, chunk tables and,
 * if built, the transpose; each array 256-byte aligned). */
ga_status graph_attn_plan_device_bytes(const ga_plan* plan, size_t* bytes);

/* Copy the plan to caller-owned device memory `dev_buf` (256-byte aligned, `bytes` >=
 * graph_attn_plan_device_bytes) with hipMemcpyAsync on `stream`, then wait for the copy.
 * The plan keeps pointers into dev_buf: the buffer must outlive every fwd/bwd call that
 * uses the plan. Uploading again re-targets the plan to the new buffer. */
ga_status graph_attn_plan_upload(ga_plan* plan, void* dev_buf, size_t bytes, void* stream);

/* Host views of the plan's arrays, for tests and tools. Names: "indptr", "indices",
 * "row_light", "row_medium", "row_hub", "row_chunk_row", "row_chunk_begin",
 * "row_chunk_end", "row_hub_chunk_ptr", and with the transpose "colptr", "rowidx",
 * "col_light", "col_medium", "col_hub", "col_chunk_row", "col_chunk_begin",
 * "col_chunk_end", "col_hub_chunk_ptr", "csc_rel", then "row_sched" and "col_sched"
 * (the latter needs the transpose). *data stays valid until the plan is
 * destroyed (it may be NULL when *count == 0). GA_ERR_INVALID_ARG for an unknown name,
 * GA_ERR_NOT_READY for a transpose array of a plan built without it. */
ga_status graph_attn_plan_array(const ga_plan* plan, const char* name, const int32_t** data,
                                int64_t* count);

/* Number of exported array names and the i-th name (NULL if out of range). */
int32_t graph_attn_plan_array_count(void);
const char* graph_attn_plan_array_name(int32_t index);

/* Release a plan's host memory (the caller frees the device copy). NULL is a no-op. */
void graph_attn_plan_destroy(ga_plan* plan);

/* Workspace the forward needs: fp32 (m, l, acc) partial states of the hub-row chunks,
 * n_row_chunks * (H*d + 2*H) * 4 bytes, 256-byte aligned sections (0 if no hub rows). */
ga_status graph_attn_fwd_workspace_bytes(const ga_plan* plan, int32_t heads, int32_t dim,
                                         size_t* bytes);

/* Forward (Methodology, attention-based layers, forward pass: fused score -> online
 * softmax -> weighted value sum; per-node log-sum-exp kept for the backward).
 *   dot: q_or_s = q, k_or_t = k, both [N,H,d] of `dtype`;  gat: q_or_s = s,
 *   k_or_t = t, both fp32 [N,H]. v [N,H,d] of `dtype`. out [N,H,d] of `dtype` (bf16 by
 *   round-to-nearest-even), lse fp32 [N,H] (natural log). scale multiplies the score
 *   (1/sqrt(d) is the usual dot value, 1 the GAT value); neg_slope is the LeakyReLU
 *   slope (gat only). workspace: graph_attn_fwd_workspace_bytes bytes (NULL allowed when
 *   that is 0). All computation in fp32. The plan must be uploaded. */
ga_status graph_attn_fwd(const ga_plan* plan, ga_score score, ga_dtype dtype, int32_t heads,
                         int32_t dim, float scale, float neg_slope, const void* q_or_s,
                         const void* k_or_t, const void* v, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same computation, arguments, kernels and results (bit for bit) as
 * graph_attn_fwd, without the workspace arguments: the hub-chunk partial states go to a
 * scratch array of GA_FWD_NOALLOC_SCRATCH_BYTES that the library holds in device memory,
 * one per GPU, from the first such call on that GPU until the process ends. A call whose
 * graph_attn_fwd_workspace_bytes exceeds that size is rejected with GA_ERR_TOO_LARGE
 * before any HIP call. Calls never allocate, free or memset device memory; each GPU's
 * scratch keeps the last call's partials (every partial a call reads it writes first, so
 * nothing needs clearing). All calls on one GPU share its scratch: calls that may overlap
 * on one GPU (different streams, or different host threads) race and must be serialised
 * by the caller; calls on one stream are ordered by the stream. */
#define GA_FWD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ga_status graph_attn_fwd_noalloc(const ga_plan* plan, ga_score score, ga_dtype dtype,
                                 int32_t heads, int32_t dim, float scale, float neg_slope,
                                 const void* q_or_s, const void* k_or_t, const void* v, void* out,
                                 float* lse, void* stream);

/* GATv2 forward (the GATv2 layer the Methodology names; the textbook score, not printed on
 * the pages): per head h,
 *     e_ij = scale * sum_c attn[h,c] * LeakyReLU_{neg_slope}(xd[i,h,c] + xs[j,h,c])
 *     out[i,h,:] = sum_j softmax_j(e_ij) xs[j,h,:],   lse[i,h] = ln sum_j exp(e_ij)
 * xd (destination projection) and xs (source projection, also the message) are [N,H,d] of
 * `dtype`; attn is fp32 [H,d] (16-byte aligned); out, lse and the workspace as for
 * graph_attn_fwd (same workspace size). Each edge gathers one source row. */
ga_status graph_attn_fwd_gatv2(const ga_plan* plan, ga_dtype dtype, int32_t heads, int32_t dim,
                               float scale, float neg_slope, const void* xd, const void* xs,
                               const float* attn, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Workspace the backward needs (either score): per-node (lse*log2 e, D) records N*H*8
 * bytes, fp32 row-chunk partials n_row_chunks*(2*H*d + 4*ceil(2H/4))*4 bytes and fp32
 * column-chunk partials n_col_chunks*2*H*d*4 bytes, each section 256-byte aligned. */
ga_status graph_attn_bwd_workspace_bytes(const ga_plan* plan, int32_t heads, int32_t dim,
                                         size_t* bytes);

/* Backward by recomputation (Methodology, attention-based layers, backward pass: attention
 * weights recomputed from the cached per-node log-sum-exp). With P_ij = exp(e_ij - lse_i),
 * dp_ij = <dout_i, v_j>, D_i = sum_j P_ij dp_ij (per head), dS_ij = P_ij (dp_ij - D_i):
 *   dot: dq_i = scale sum_j dS_ij k_j             (over CSR rows)
 *        dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dout_i   (over the transpose)
 *   gat: with x_ij = s_i + t_j and g_ij = 1 if x_ij >= 0 else neg_slope,
 *        ds_i = scale sum_j dS_ij g_ij             (over CSR rows)
 *        dt_j = scale sum_i dS_ij g_ij,  dv_j = sum_i P_ij dout_i   (over the transpose)
 * D_i is accumulated in the row pass from the recomputed weights, so the forward output
 * is not needed; the row pass also sums the recomputed weights (1 up to the rounding of
 * the stored lse) and divides by that sum, so both passes use weights that sum to 1.
 * Arguments by score:
 *   dot: q, k, v, dout, dq, dk, dv are [N,H,d] of `dtype` (16-byte aligned).
 *   gat: q = s, k = t, dq = ds, dk = dt are fp32 [N,H] (4-byte aligned); v, dout, dv are
 *        [N,H,d] of `dtype`. neg_slope is the forward's LeakyReLU slope (ignored for dot).
 * lse: fp32 [N,H] as produced by graph_attn_fwd with the same scale (and slope). Every
 * output is fully written (rows and columns with no edges get zeros). Needs a plan built
 * with build_csc and uploaded (else GA_ERR_NOT_READY). */
ga_status graph_attn_bwd(const ga_plan* plan, ga_score score, ga_dtype dtype, int32_t heads,
                         int32_t dim, float scale, float neg_slope, const void* q,
                         const void* k, const void* v, const void* dout, const float* lse,
                         void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Workspace of graph_attn_bwd_gatv2: per-node records N*H*8 bytes, row-chunk partials
 * n_row_chunks*(2*H*d + 4*ceil(2H/4))*4, column-chunk partials n_col_chunks*2*H*d*4, the
 * attention-gradient partials (S = one per 16 work items of the row pass, one per 16 of the
 * column pass, plus one per hub row and hub column, H*d*4 bytes each) and fp64 reduction buffers
 * of (ceil(S/32) + ceil(S/1024))*H*d*8
 * bytes, each section 256-byte aligned (0 bytes for a graph with no nodes: then the
 * workspace may be NULL). The number of work items depends on the lanes per feature row,
 * hence `dtype`. */
ga_status graph_attn_bwd_gatv2_workspace_bytes(const ga_plan* plan, ga_dtype dtype,
                                               int32_t heads, int32_t dim, size_t* bytes);

/* GATv2 backward by recomputation. With z_ij = xd_i + xs_j, g = LeakyReLU'(z) (1 where
 * z >= 0, else neg_slope, elementwise), P_ij = exp(e_ij - lse_i), dp_ij = <dout_i, xs_j>,
 * D_i = sum_j P_ij dp_ij and dS_ij = P_ij (dp_ij - D_i):
 *     dxd_i = scale * attn (.) sum_j dS_ij g_ij
 *     dxs_j = scale * attn (.) sum_i dS_ij g_ij + sum_i P_ij dout_i
 *     dattn = scale * sum_(i,j) dS_ij LeakyReLU(z_ij)     (fp32 [H,d])
 * Rows are renormalised as in graph_attn_bwd. xd, xs, dout, dxd, dxs are [N,H,d] of
 * `dtype` (16-byte aligned); attn and dattn fp32 [H,d] (16-byte aligned). dattn is reduced
 * in a fixed order (fp64 final stages), so results are bitwise reproducible. Needs a plan
 * with the transpose, uploaded. */
ga_status graph_attn_bwd_gatv2(const ga_plan* plan, ga_dtype dtype, int32_t heads, int32_t dim,
                               float scale, float neg_slope, const void* xd, const void* xs,
                               const float* attn, const void* dout, const float* lse, void* dxd,
                               void* dxs, float* dattn, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ---- Neighbourhood reduction (min / max pooling) -------------------------------------
 * The reduction-based layer family of the same pages (Technical Summary > Methodology,
 * reduction-based layers: a per-edge message reduced over each node's neighbourhood by
 * min or max, rows split by degree into light rows handled feature-parallel and heavy
 * rows reduced as parallel edge chunks whose partial results combine as (value, index)
 * pairs). The message of edge (i <- j) is the source row x[j] itself; every one of the
 * F feature elements is reduced separately:
 *     out[i,c] = max_j x[j,c]  (or min)     arg[i,c] = the source id j attaining it
 * Equal values go to the smallest source id, so arg does not depend on the order of a
 * row's neighbours. out[i,c] is x[arg[i,c],c] bit for bit (values compare as numbers:
 * -0 equals +0). A row with no neighbours gives out = 0 and arg = -1. Optionally the
 * forward also writes slot[i,c] = the position within row i (k - indptr[i]) of the first
 * edge of that row from arg[i,c], in the plan's CSR (the caller's, unless the plan has an
 * XCD split, which regroups long rows: see graph_attn_plan_array "indices"), as unsigned 16-bit values when no row has more than
 * 65535 edges, else 32-bit (graph_attn_reduce_slot_bytes); an element without a winner
 * (an empty row) gets all ones, which no position equals. The
 * backward reads slot (2 bytes per element per transpose edge) in place of arg (4), so a
 * training step should keep slot. NaN never wins a
 * comparison (a row whose candidates are all NaN reads as empty); inputs are meant to be
 * free of NaN. x, out, dout, dx: [N, F] of `dtype`, F*sizeof(dtype) one of 64, 128, 256,
 * 512 or 1024 bytes; arg int32 [N, F]; every pointer 16-byte aligned. Results are
 * bitwise reproducible (no atomics; the backward's sums run in a fixed order). */
typedef enum { GA_REDUCE_MAX = 0, GA_REDUCE_MIN = 1 } ga_reduce;

/* Workspace of graph_attn_reduce_fwd: per hub-row chunk, the fp32 values, int32 ids and
 * int32 edge indices of its partial result, three sections of n_row_chunks*F*4 bytes,
 * each 256-byte aligned (0 when the plan has no hub rows; the workspace may then be
 * NULL). */
ga_status graph_attn_reduce_fwd_workspace_bytes(const ga_plan* plan, int32_t features,
                                                size_t* bytes);

/* Bytes per element of the plan's slot array: 2 when no row has more than 65535 edges,
 * else 4. */
ga_status graph_attn_reduce_slot_bytes(const ga_plan* plan, size_t* bytes);

/* Forward: out and arg for every row, and slot when `slot` is not NULL ([N, F] of
 * graph_attn_reduce_slot_bytes each, 16-byte aligned). The plan must be uploaded. */
ga_status graph_attn_reduce_fwd(const ga_plan* plan, ga_reduce op, ga_dtype dtype,
                                int32_t features, const void* x, void* out, int32_t* arg,
                                void* slot, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Workspace of graph_attn_reduce_bwd: fp32 partial sums of the hub-column chunks,
 * n_col_chunks*F*4 bytes (0 when the transpose has no hub columns; NULL allowed then). */
ga_status graph_attn_reduce_bwd_workspace_bytes(const ga_plan* plan, int32_t features,
                                                size_t* bytes);

/* Backward: dx[j,c] = sum of dout[i,c] over the destinations i with arg[i,c] = j (each
 * distinct i once; a parallel edge does not count twice), the gradient of the forward
 * routed to the element that won. Pass the forward's slot (then arg may be NULL and is not
 * read) or, without slot, its arg. Both are only compared with column ids or transpose
 * positions, never used as addresses, so an entry that is neither matches nothing.
 * Computed over the plan's cached transpose, one pass per source column, sums in fp32
 * (fp64 when dtype is fp32) in a fixed order. Needs a plan with the transpose, uploaded. */
ga_status graph_attn_reduce_bwd(const ga_plan* plan, ga_dtype dtype, int32_t features,
                                const int32_t* arg, const void* slot, const void* dout,
                                void* dx, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Kernel timers (tracing). When enabled, every kernel the library launches is bracketed
 * by two hipEvents recorded on its stream; graph_attn_timer_read synchronises those
 * events and reports, per kernel name, the number of launches and their summed duration
 * in milliseconds. Process-wide, thread-safe. Disabled by default. */
ga_status graph_attn_timer_enable(int32_t enable);
ga_status graph_attn_timer_reset(void);
/* Number of distinct kernel names recorded since the last reset. */
int32_t graph_attn_timer_count(void);
/* The index-th record: name (static string), launches and total milliseconds. */
ga_status graph_attn_timer_read(int32_t index, const char** name, int64_t* launches,
                                double* total_ms);

/* Device-to-device copy of `bytes` bytes with the library's streaming copy kernel (16-byte
 * vector loads/stores). Both pointers 16-byte aligned, bytes a multiple of 16. Used to
 * measure copy bandwidth and to calibrate traffic counters against a known byte count. */
ga_status graph_attn_copy_probe(void* dst, const void* src, size_t bytes, void* stream);

/* Gather-only probes: the loads of an attention pass with its arithmetic taken out, on
 * the same plan and in the same order (work items, lanes of 16 bytes, edges in flight),
 * folded into an XOR so they stay live, with no stores (but an improbable one to `sink`).
 * Their durations bound the passes' times from below on that graph: the time the memory
 * system takes to deliver the pass's reads. sink: 1 KiB of device memory, 16-byte aligned.
 * Rows, dtype and geometry as for graph_attn_fwd; pointers that may be NULL mean "not
 * read". The plan must be uploaded (and, for the columns probe, built with the transpose).
 *
 * graph_attn_gather_probe: the work list of graph_attn_fwd and of the backward's dQ pass:
 * the plan's hub-chunk slots (in its XCD schedule), medium rows, then light rows, with the
 * forward's feature slices. Per work item it reads row_a[i] and row_b[i] (the row-side
 * operands: q for the forward, q and dout for the dQ pass; either may be NULL); per edge
 * (i <- j) k[j] and v[j] (v NULL: one row per edge, as the GATv2 forward gathers). */
ga_status graph_attn_gather_probe(const ga_plan* plan, ga_dtype dtype, int32_t heads,
                                  int32_t dim, const void* row_a, const void* row_b,
                                  const void* k, const void* v, void* sink, void* stream);

/* graph_attn_gather_probe_cols: the work list of the backward's dK/dV pass over the
 * transpose: hub-column chunk slots (in the plan's column XCD schedule), medium columns,
 * then light columns. Per column j it reads k[j] and v[j] (either may be NULL); per
 * transpose edge (i -> j) dout[i], q[i] (q may be NULL) and the fp32 (lse, D) record
 * pair of i's head, record [N, heads, 2] (may be NULL; 8-byte aligned). */
ga_status graph_attn_gather_probe_cols(const ga_plan* plan, ga_dtype dtype, int32_t heads,
                                       int32_t dim, const void* k, const void* v, const void* q,
                                       const void* dout, const float* record, void* sink,
                                       void* stream);

/* graph_attn_gather_probe_random: n_gathers rows of row_bytes bytes (64, 128, 256, 512 or
 * 1024) drawn uniformly at random from a table of table_rows rows (1 <= table_rows <
 * 2^32; the table holds table_rows * row_bytes bytes, 16-byte aligned), gather k reading
 * the row picked by the k-th output of the SplitMix64 generator seeded with `seed`; 16 bytes
 * per lane, 8 rows in flight per lane group. Its rate at a given table size is the gather
 * ceiling of the memory hierarchy at that footprint (L2, the MALL, HBM). Needs no plan. */
ga_status graph_attn_gather_probe_random(int32_t row_bytes, const void* table,
                                         int64_t table_rows, int64_t n_gathers, uint64_t seed,
                                         void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GRAPH_ATTN_H */
