// Forward kernels of fused CSR graph attention for gfx950.
//
// Method: "On Efficient Scaling of GNNs via IO-Aware Layers Implementations", Technical
// Summary > Methodology, attention-based layers, forward pass: score computation, softmax
// normalisation and value aggregation fused in one streaming pass over a row's
// neighbours, with the running softmax statistics held in registers (online softmax), so
// no edge-wise logits are materialised. Degree-aware work split after the same section's
// reduction paragraph (light rows feature-parallel, heavy rows as parallel edge chunks).
//
// One launch (fwd_main) covers every row. Its wavefront work items are, in order:
//   [0, n_sched)                 hub-row chunks: one wavefront per chunk -> fp32 partial
//                                (m, l, acc) in the workspace; slot k runs chunk k, or
//                                the chunk the plan's XCD schedule puts there (none: -1)
//   [.., + n_medium)             medium rows: one wavefront per row
//   [.., + ceil(n_light / NG))   light rows: one G-lane group per row, NG rows per wave
// Bins are sorted by degree descending, so the longest items start first. A second
// launch (fwd_hub_merge) folds each hub row's chunk partials in ascending chunk order.
// With feature slices (see fwd_main) every item is run once per slice of whole heads, the
// slices dealt to XCD groups; the merge works on full rows.
//
// Score modes: dot (q_i . k_j), GAT-style (LeakyReLU(s_i + t_j)) and GATv2
// (a . LeakyReLU(xd_i + xs_j), where the gathered source row xs_j is also the value, so a
// GATv2 edge gathers one row instead of two).
//
// Per edge a lane group gathers the neighbour's K and V rows with 16-byte loads per lane
// (coalesced across the group; structured buffer loads that take the node id, or plain
// 64-bit loads for tables past 4 GiB), reduces the per-head dot product with DPP adds,
// and folds U edges at a time into the running (m, l, acc) state: one rescale per U
// edges. Scores are kept in log2 units (scale * log2 e folded into one multiplier) so every
// exponential is a single v_exp_f32. No atomics: results are bitwise reproducible.
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {
namespace {

// LeakyReLU with slope s as alpha z + beta |z|, alpha = (1 + s) / 2, beta = (1 - s) / 2: the
// two forms agree for either sign of z and any s, so a . LeakyReLU(z) is alpha a . z +
// beta a . |z|, two FMAs per element (|z| is a free source modifier) and no compare or
// select.
struct LeakySplit {
  float alpha, beta;
};
__device__ __forceinline__ LeakySplit leaky_split(float slope) {
  return {0.5f * (1.f + slope), 0.5f * (1.f - slope)};
}

template <typename T, int G, int LH, int MODE, int U>
struct Fwd {
  static constexpr bool GAT = MODE == kModeGat;
  static constexpr bool GATV2 = MODE == kModeGatV2;
  using L16 = Lane16<T>;
  using raw_t = typename L16::raw_t;
  static constexpr int VEC = L16::VEC;
  static constexpr int NG = kWave / G;  // lane groups per wavefront
  static constexpr int H = G / LH;      // heads
  static constexpr int F = G * VEC;     // elements per feature row

  struct State {
    float m, l;
    float acc[VEC];
  };

  __device__ __forceinline__ static void init(State& s) {
    s.m = kEmptyMax;
    s.l = 0.f;
#pragma unroll
    for (int c = 0; c < VEC; ++c) s.acc[c] = 0.f;
  }

  // Row-side operand of the score: the query row slice (dot), s[i, h] (gat), or the
  // destination projection xd_i plus the lane's slice of the attention vector and the two
  // halves of the LeakyReLU split (gatv2; see leaky_split).
  struct RowOp {
    raw_t q;
    float si;
    float xd[GATV2 ? VEC : 1];
    float av[GATV2 ? VEC : 1];
    LeakySplit ls;
  };

  __device__ __forceinline__ static void load_row(const FwdArgs& a, int row, int r, int h,
                                                  RowOp& q) {
    if constexpr (GAT) {
      q.si = ld_stream(static_cast<const float*>(a.a) + static_cast<size_t>(row) * a.hf + h);
    } else {
      q.q = ld_stream(static_cast<const raw_t*>(a.a) + static_cast<size_t>(row) * a.ld + r);
    }
    if constexpr (GATV2) {
      L16::unpack(q.q, q.xd);
      q.ls = leaky_split(a.neg_slope);
      const f32x4* ap = reinterpret_cast<const f32x4*>(a.attn + r * VEC);
#pragma unroll
      for (int k = 0; k < VEC / 4; ++k) {
        const f32x4 x = ap[k];
        q.av[4 * k] = x.x;
        q.av[4 * k + 1] = x.y;
        q.av[4 * k + 2] = x.z;
        q.av[4 * k + 3] = x.w;
      }
    }
  }

  // Stream edges [e0, e1) through the state with NGS lane groups cooperating. seg0 is the
  // segment's first lane in the wave, gs this lane's group within the segment. WIDE: the
  // gathered tables are larger than one 4 GiB buffer window (FwdArgs::wide).
  template <int NGS, bool WIDE>
  __device__ __forceinline__ static void run(const FwdArgs& a, int e0, int e1, int seg0, int gs,
                                             int r, int h, const RowOp& q, State& st) {
    constexpr int L = NGS * G;  // lanes of the segment = indices fetched per batch
    const int lane = threadIdx.x & (kWave - 1);
    // K and V rows through structured buffers (plain loads for tables past 4 GiB); GAT's t
    // entries (4 bytes per head, read by every lane of the head) by plain loads, which serve
    // that pattern faster
    const rows_t Kd = node_rows(a.b, a.ld * int(sizeof(raw_t)), a.n);
    const rows_t Vd = node_rows(a.v, a.ld * int(sizeof(raw_t)), a.n);
    const raw_t* __restrict__ Kr = static_cast<const raw_t*>(a.b);
    const raw_t* __restrict__ Vr = static_cast<const raw_t*>(a.v);
    const float* __restrict__ Tt = static_cast<const float*>(a.b);
    for (int base = e0; base < e1; base += L) {
      const int nb = min(L, e1 - base);
      const int li = lane - seg0;
      // lanes past the batch's edges name node n, one past the table: a structured buffer
      // load out of range returns zeros without touching memory. A step's spare slots read
      // those lanes or, where a step is longer than a batch, lanes of the same batch (edges
      // of this row, weighted zero), so what a table holds outside this row's neighbours
      // never enters the sums. Plain 64-bit loads have no range check; there the spare
      // lanes name the batch's first edge, a neighbour of the same row.
      const int my_j = WIDE ? ld_stream(a.indices + base + (li < nb ? li : 0))
                            : (li < nb ? ld_stream(a.indices + base + li) : a.n);
      for (int t = 0; t < nb; t += NGS * U) {
        int jj[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int pos = t + u * NGS + gs;
          ok[u] = pos < nb;
          jj[u] = __builtin_amdgcn_ds_bpermute((seg0 + pos) << 2, my_j);
        }
        raw_t kr[U], vr[U];
        float tv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if constexpr (GAT)
            tv[u] = Tt[static_cast<size_t>(min(jj[u], a.n - 1)) * a.hf + h];  // plain load: in range
          else
            kr[u] = ld_node<WIDE>(Kd, Kr, jj[u], a.ld, r);
          if constexpr (GATV2)
            vr[u] = kr[u];  // the message is the gathered source projection
          else
            vr[u] = ld_node<WIDE>(Vd, Vr, jj[u], a.ld, r);
        }
        float s[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float x;
          if constexpr (GAT) {
            x = q.si + tv[u];
            x = (x >= 0.f ? x : x * a.neg_slope) * a.sc2;
          } else if constexpr (GATV2) {
            float xs[VEC];
            L16::unpack(kr[u], xs);
            // a . LeakyReLU(z) = alpha a . z + beta a . |z|: two FMAs per element
            float e1 = 0.f, e2 = 0.f;
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
              const float z = q.xd[c] + xs[c];
              e1 = fmaf(q.av[c], z, e1);
              e2 = fmaf(q.av[c], fabsf(z), e2);
            }
            x = head_sum<LH>(fmaf(q.ls.alpha, e1, q.ls.beta * e2)) * a.sc2;
          } else {
            x = head_sum<LH>(L16::dot(q.q, kr[u])) * a.sc2;
          }
          s[u] = ok[u] ? x : -INFINITY;
        }
        float mt = s[0];
#pragma unroll
        for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u]);
        const float mn = fmaxf(st.m, mt);
        const float corr = fast_exp2(st.m - mn);
        st.l *= corr;
#pragma unroll
        for (int c = 0; c < VEC; ++c) st.acc[c] *= corr;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float p = fast_exp2(s[u] - mn);
          float vf[VEC];
          L16::unpack(vr[u], vf);
          st.l += p;
#pragma unroll
          for (int c = 0; c < VEC; ++c) st.acc[c] = fmaf(p, vf[c], st.acc[c]);
        }
        st.m = mn;
      }
    }
  }

  // Fold the states of the NGS groups of a segment (butterfly over lane distance G..).
  template <int NGS>
  __device__ __forceinline__ static void combine(State& st) {
#pragma unroll
    for (int off = G; off < NGS * G; off <<= 1) {
      const float m2 = __shfl_xor(st.m, off);
      const float l2 = __shfl_xor(st.l, off);
      const float mn = fmaxf(st.m, m2);
      const float c1 = fast_exp2(st.m - mn);
      const float c2 = fast_exp2(m2 - mn);
      st.l = st.l * c1 + l2 * c2;
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        const float a2 = __shfl_xor(st.acc[c], off);
        st.acc[c] = st.acc[c] * c1 + a2 * c2;
      }
      st.m = mn;
    }
  }

  __device__ __forceinline__ static void write_row(const FwdArgs& a, int row, int r, int h,
                                                   const State& st) {
    const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
    float o[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) o[c] = st.acc[c] * inv;
    st_stream(static_cast<raw_t*>(a.out) + static_cast<size_t>(row) * a.ld + r, L16::pack(o));
    if (r % LH == 0)
      st_stream(a.lse + static_cast<size_t>(row) * a.hf + h,
                st.l > 0.f ? (st.m + __log2f(st.l)) * kLn2 : -INFINITY);
  }

  __device__ __forceinline__ static void write_partial(const FwdArgs& a, int chunk, int r, int h,
                                                       const State& st) {
    if (r % LH == 0) {
      f32x2* ml = reinterpret_cast<f32x2*>(a.ws_ml);
      st_stream(ml + static_cast<size_t>(chunk) * a.hf + h, f32x2{st.m, st.l});
    }
    f32x4* acc = reinterpret_cast<f32x4*>(a.ws_acc + static_cast<size_t>(chunk) * a.ld * VEC +
                                          r * VEC);
#pragma unroll
    for (int c = 0; c < VEC / 4; ++c)
      st_stream(acc + c, f32x4{st.acc[4 * c], st.acc[4 * c + 1], st.acc[4 * c + 2],
                               st.acc[4 * c + 3]});
  }
};

// The GATv2 score gathers one row per edge and is paced by its per-edge arithmetic and the
// latency of the gathers that feed it; it trades edges per step for waves per SIMD:
// 4 edges per step (2 in light rows) fit in at most 80 VGPRs, six waves, with no spills.
#ifndef GA_UNROLL_FWD_GATV2
#define GA_UNROLL_FWD_GATV2 4
#endif
#ifndef GA_UNROLL_FWD_GATV2_LIGHT
#define GA_UNROLL_FWD_GATV2_LIGHT 2
#endif
#ifndef GA_WAVES_FWD_GATV2
#define GA_WAVES_FWD_GATV2 6
#endif

// Waves per SIMD the register allocator must make room for: GA_WAVES_FWD_GATV2 for the
// GATv2 score; the dot and GAT-style scores take GA_WAVES_PER_EU, or the compiler's own
// choice (1 sets no floor).
template <int MODE>
constexpr int fwd_min_waves() {
  return MODE == kModeGatV2 ? GA_WAVES_FWD_GATV2 : (GA_WAVES_PER_EU > 0 ? GA_WAVES_PER_EU : 1);
}

// A "slice" is G lanes (whole heads) of a feature row of a.ld lanes; the kernel's template
// geometry is the slice's. slice_of() deals slices to XCDs (see ga_device.h); each wave
// moves its operand pointers to its slice, after which row strides (a.ld lanes, a.hf
// heads) address the full rows.
template <typename T, int G, int LH, int MODE, int U, int UL, bool WIDE>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(fwd_min_waves<MODE>())))
void fwd_main(FwdArgs a0) {
  using K = Fwd<T, G, LH, MODE, U>;
  using KL = Fwd<T, G, LH, MODE, UL>;  // light rows
  using raw_t = typename K::raw_t;
  constexpr int NG = K::NG, H = K::H, VEC = K::VEC;
  const int lane = threadIdx.x & (kWave - 1);
  const SliceItem si = slice_of(a0.slices);
  const int item = si.item;
  FwdArgs a = a0;
  {
    const int so = si.slice * G, ho = si.slice * H;  // lanes / heads before this slice
    if constexpr (MODE == kModeGat) {
      a.a = static_cast<const float*>(a0.a) + ho;
      a.b = static_cast<const float*>(a0.b) + ho;
    } else {
      a.a = static_cast<const raw_t*>(a0.a) + so;
      a.b = static_cast<const raw_t*>(a0.b) + so;
    }
    a.v = static_cast<const raw_t*>(a0.v) + so;
    a.out = static_cast<raw_t*>(a0.out) + so;
    a.lse = a0.lse + ho;
    if (a0.attn) a.attn = a0.attn + so * VEC;
    a.ws_ml = a0.ws_ml + 2 * ho;
    a.ws_acc = a0.ws_acc + so * VEC;
  }
  const int g = lane / G, r = lane % G, h = r / LH;
  const DevBins& B = a.bins;
  if (item < B.n_sched + B.n_medium) {
    typename K::State st;
    typename K::RowOp q;
    K::init(st);
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
    K::load_row(a, row, r, h, q);
    K::template run<NG, WIDE>(a, e0, e1, 0, g, r, h, q, st);
    K::template combine<NG>(st);
    if (g != 0) return;
    if (chunk)
      K::write_partial(a, c, r, h, st);
    else
      K::write_row(a, row, r, h, st);
    return;
  }
  const int li = (item - B.n_sched - B.n_medium) * NG + g;
  if (li >= B.n_light) return;
  const int row = B.light[li];
  const int e0 = a.indptr[row], e1 = a.indptr[row + 1];
  typename KL::State st;
  typename KL::RowOp q;
  KL::init(st);
  KL::load_row(a, row, r, h, q);
  KL::template run<1, WIDE>(a, e0, e1, g * G, 0, r, h, q, st);
  KL::write_row(a, row, r, h, st);
}

// One wavefront per hub row: lane group g folds chunks c0+g, c0+g+NG, ... in ascending
// order, then the NG group states are combined by the fixed butterfly (deterministic).
template <typename T, int G, int LH>
__global__ __launch_bounds__(kBlock) void fwd_hub_merge(FwdArgs a) {
  using K = Fwd<T, G, LH, kModeDot, 1>;
  constexpr int VEC = K::VEC, NG = K::NG;
  const int hub = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane / G, r = lane % G, h = r / LH;
  if (hub >= a.bins.n_hub) return;
  const int row = a.bins.hub[hub];
  const int c0 = a.bins.hub_chunk_ptr[hub], c1 = a.bins.hub_chunk_ptr[hub + 1];
  const f32x2* ml = reinterpret_cast<const f32x2*>(a.ws_ml);
  typename K::State st;
  K::init(st);
#pragma unroll 4
  for (int c = c0 + g; c < c1; c += NG) {
    const f32x2 p = ld_stream(ml + static_cast<size_t>(c) * a.hf + h);
    const f32x4* acc =
        reinterpret_cast<const f32x4*>(a.ws_acc + static_cast<size_t>(c) * a.ld * VEC + r * VEC);
    f32x4 x[VEC / 4];
#pragma unroll
    for (int k = 0; k < VEC / 4; ++k) x[k] = ld_stream(acc + k);
    const float mn = fmaxf(st.m, p.x);
    const float f1 = fast_exp2(st.m - mn);
    const float f2 = fast_exp2(p.x - mn);
    st.l = st.l * f1 + p.y * f2;
#pragma unroll
    for (int k = 0; k < VEC / 4; ++k) {
      st.acc[4 * k] = st.acc[4 * k] * f1 + x[k].x * f2;
      st.acc[4 * k + 1] = st.acc[4 * k + 1] * f1 + x[k].y * f2;
      st.acc[4 * k + 2] = st.acc[4 * k + 2] * f1 + x[k].z * f2;
      st.acc[4 * k + 3] = st.acc[4 * k + 3] * f1 + x[k].w * f2;
    }
    st.m = mn;
  }
  K::template combine<NG>(st);
  if (g == 0) K::write_row(a, row, r, h, st);
}

// Main kernel on the slice geometry (G lanes per slice), a.slices slices.
template <typename T, int G, int LH, int MODE>
int launch_main(const FwdArgs& a, void* stream, TimerHook hook) {
  constexpr bool V2 = MODE == kModeGatV2;
  constexpr int U = V2 ? GA_UNROLL_FWD_GATV2 : GA_UNROLL_FWD;
  constexpr int UL = V2 ? GA_UNROLL_FWD_GATV2_LIGHT : GA_UNROLL_FWD_LIGHT;
  constexpr int NG = kWave / G;
  const DevBins& B = a.bins;
  const int64_t items = int64_t(B.n_sched) + B.n_medium + (int64_t(B.n_light) + NG - 1) / NG;
  if (items <= 0) return 0;
  const int64_t blocks = slice_blocks((items + kWavesPerBlock - 1) / kWavesPerBlock, a.slices);
  if (hook) hook("fwd_main", stream, 1);
  if (a.wide)
    hipLaunchKernelGGL((fwd_main<T, G, LH, MODE, U, UL, true>),
                       dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL((fwd_main<T, G, LH, MODE, U, UL, false>),
                       dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), a);
  if (hook) hook("fwd_main", stream, 0);
  return static_cast<int>(hipGetLastError());
}

// Hub merge on the full row geometry.
template <typename T, int G, int LH>
int launch_merge(const FwdArgs& a, void* stream, TimerHook hook) {
  const DevBins& B = a.bins;
  if (B.n_hub <= 0) return 0;
  const int blocks = (B.n_hub + kWavesPerBlock - 1) / kWavesPerBlock;
  if (hook) hook("fwd_hub_merge", stream, 1);
  hipLaunchKernelGGL((fwd_hub_merge<T, G, LH>), dim3(blocks), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), a);
  if (hook) hook("fwd_hub_merge", stream, 0);
  return static_cast<int>(hipGetLastError());
}

// (G, LH) pairs with compiled kernels: rows of 64..1024 bytes, heads of 32..1024 bytes.
#define GA_GEOMS(X)                                                                       \
  X(4, 2) X(4, 4) X(8, 2) X(8, 4) X(8, 8) X(16, 2) X(16, 4) X(16, 8) X(16, 16) X(32, 2) \
  X(32, 4) X(32, 8) X(32, 16) X(32, 32) X(64, 2) X(64, 4) X(64, 8) X(64, 16) X(64, 32) \
  X(64, 64)

template <typename T, int MODE>
int dispatch(const Geometry& g, const FwdArgs& a, void* stream, TimerHook hook) {
  const int GS = g.G / a.slices;
  int e = -1;
#define GA_CASE(GG, LL) \
  if (GS == GG && g.LH == LL) e = launch_main<T, GG, LL, MODE>(a, stream, hook);
  GA_GEOMS(GA_CASE)
#undef GA_CASE
  if (e) return e;
#define GA_CASE(GG, LL) \
  if (g.G == GG && g.LH == LL) return launch_merge<T, GG, LL>(a, stream, hook);
  GA_GEOMS(GA_CASE)
#undef GA_CASE
  return -1;
}

bool geom_ok(const Geometry& g) {
#define GA_CASE(GG, LL) \
  if (g.G == GG && g.LH == LL) return true;
  GA_GEOMS(GA_CASE)
#undef GA_CASE
  return false;
}

}  // namespace

bool fwd_supported(ga_dtype dt, ga_score sc, const Geometry& g) {
  return (dt == GA_F32 || dt == GA_BF16) && (sc == GA_SCORE_DOT || sc == GA_SCORE_GAT) &&
         geom_ok(g);
}

template <typename T>
int dispatch_mode(int mode, const Geometry& g, const FwdArgs& a, void* stream, TimerHook hook) {
  switch (mode) {
    case kModeDot: return dispatch<T, kModeDot>(g, a, stream, hook);
    case kModeGat: return dispatch<T, kModeGat>(g, a, stream, hook);
    case kModeGatV2: return dispatch<T, kModeGatV2>(g, a, stream, hook);
  }
  return -1;
}

int launch_fwd(ga_dtype dt, int mode, const Geometry& g, const FwdArgs& a, int64_t,
               void* stream, TimerHook hook) {
  return dt == GA_F32 ? dispatch_mode<float>(mode, g, a, stream, hook)
                      : dispatch_mode<bf16_t>(mode, g, a, stream, hook);
}

}  // namespace ga
