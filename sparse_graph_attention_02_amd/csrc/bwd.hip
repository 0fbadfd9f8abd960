// Backward kernels of fused CSR graph attention (dot score) for gfx950.
//
// Method: "On Efficient Scaling of GNNs via IO-Aware Layers Implementations", Technical
// Summary > Methodology, attention-based layers, backward pass: only a compact per-node
// statistic (the log-sum-exp) is kept from the forward and the attention weights are
// recomputed on the fly; the transposed adjacency is precomputed once (same section, SpMM
// paragraph) so that dK/dV are gathered per source column instead of scattered with
// atomics.
//
// With P_ij = exp(e_ij - lse_i), dp_ij = <dout_i, v_j>, D_i = sum_j P_ij dp_ij (per head),
// dS_ij = P_ij (dp_ij - D_i):
//   bwd_dq_main     over CSR rows (same bins / item order as the forward), one pass:
//                   L_i = sum_j P_ij, A_i = sum_j P_ij dp_ij k_j, B_i = sum_j P_ij k_j,
//                   D_i = sum_j P_ij dp_ij. L is 1 up to the rounding of the stored lse;
//                   dividing by it makes the recomputed weights sum to 1, so with
//                   D^ = D / L:  dq_i = scale (A_i - D^_i B_i) / L_i = scale sum_j dS_ij k_j
//                   (single-neighbour rows give dq = 0 up to one rounding). The record
//                   (lse_i log2 e + log2 L_i, D^_i) goes to the column pass, whose weights
//                   are then normalised the same way. D comes from the recomputed weights,
//                   not from the rounded stored output (hub rows: fp32 chunk partials of
//                   A, B, D, L)
//   bwd_dq_merge    hub rows: sum chunk partials in ascending chunk order
//   bwd_dkdv_main   over transpose columns (column bins by out-degree):
//                   dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dout_i
//   bwd_dkdv_merge  hub columns: sum chunk partials in ascending chunk order
// Every sum runs in fp32 in a fixed order; no atomics.
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {
namespace {

template <typename T, int G, int LH, int U>
struct Bwd : RowIO<T, G, LH> {
  using IO = RowIO<T, G, LH>;
  using typename IO::L16;
  using typename IO::raw_t;
  using IO::F;
  using IO::H;
  using IO::NG;
  using IO::R;
  using IO::VEC;
  using IO::store;
  using typename IO::acc_t;
  static constexpr int kDqStride = 2 * F + (2 * H + 3) / 4 * 4;

  // ---- dQ over CSR rows ------------------------------------------------------------
  // Accumulates A += P dp k, B += P k, D += P dp and L += P over edges [e0, e1).
  template <int NGS>
  __device__ __forceinline__ static void run_dq(const BwdArgs& a, int e0, int e1, int seg0,
                                                int gs, int r, const raw_t& qr, const raw_t& dor,
                                                float lse2, float* A, float* Bk, float& D,
                                                float& Lp) {
    constexpr int L = NGS * G;
    const int lane = threadIdx.x & (kWave - 1);
    const raw_t* __restrict__ Kr = R(a.k);
    const raw_t* __restrict__ Vr = R(a.v);
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
          jj[u] = __shfl(my_j, seg0 + (ok[u] ? pos : t));
        }
        raw_t kr[U], vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          kr[u] = Kr[static_cast<size_t>(jj[u]) * a.ld + r];
          vr[u] = Vr[static_cast<size_t>(jj[u]) * a.ld + r];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float kf[VEC];
          L16::unpack(kr[u], kf);
          const float s2 = head_sum<LH>(L16::dot(qr, kr[u])) * a.sc2;
          const float dp = head_sum<LH>(L16::dot(dor, vr[u]));
          const float p = ok[u] ? fast_exp2(s2 - lse2) : 0.f;
          const float pdp = p * dp;
          D += pdp;
          Lp += p;
#pragma unroll
          for (int c = 0; c < VEC; ++c) {
            A[c] = fmaf(pdp, kf[c], A[c]);
            Bk[c] = fmaf(p, kf[c], Bk[c]);
          }
        }
      }
    }
  }

  // ---- dK / dV over transpose columns ----------------------------------------------
  template <int NGS>
  __device__ __forceinline__ static void run_dkdv(const BwdArgs& a, int e0, int e1, int seg0,
                                                  int gs, int r, int h, const raw_t& kr,
                                                  const raw_t& vr, acc_t* dk, acc_t* dv) {
    constexpr int L = NGS * G;
    const int lane = threadIdx.x & (kWave - 1);
    const raw_t* __restrict__ Qr = R(a.q);
    const raw_t* __restrict__ Or = R(a.dout);
    const f32x2* __restrict__ LD = reinterpret_cast<const f32x2*>(a.ws_ld);
    for (int base = e0; base < e1; base += L) {
      const int nb = min(L, e1 - base);
      const int li = lane - seg0;
      const int my_i = (li < nb) ? ld_stream(a.rowidx + base + li) : 0;
      for (int t = 0; t < nb; t += NGS * U) {
        int ii[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int pos = t + u * NGS + gs;
          ok[u] = pos < nb;
          ii[u] = __shfl(my_i, seg0 + (ok[u] ? pos : t));
        }
        raw_t qr[U], dr[U];
        f32x2 ld[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          qr[u] = Qr[static_cast<size_t>(ii[u]) * G + r];
          dr[u] = Or[static_cast<size_t>(ii[u]) * G + r];
          ld[u] = LD[static_cast<size_t>(ii[u]) * H + h];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float qf[VEC], df[VEC];
          L16::unpack(qr[u], qf);
          L16::unpack(dr[u], df);
          const float s2 = head_sum<LH>(L16::dot(qr[u], kr)) * a.sc2;
          const float dp = head_sum<LH>(L16::dot(dr[u], vr));
          const float p = ok[u] ? fast_exp2(s2 - ld[u].x) : 0.f;
          const float ds = p * (dp - ld[u].y);
#pragma unroll
          for (int c = 0; c < VEC; ++c) {
            dk[c] = fma(static_cast<acc_t>(ds), static_cast<acc_t>(qf[c]), dk[c]);
            dv[c] = fma(static_cast<acc_t>(p), static_cast<acc_t>(df[c]), dv[c]);
          }
        }
      }
    }
  }

  // Row prologue of the dQ pass: q and dout slices, lse in log2 units.
  __device__ __forceinline__ static void row_prologue(const BwdArgs& a, int row, int r, int h,
                                                      raw_t& qr, raw_t& dor, float& lse2) {
    const size_t off = static_cast<size_t>(row) * a.ld + r;
    qr = ld_stream(R(a.q) + off);
    dor = ld_stream(R(a.dout) + off);
    lse2 = ld_stream(a.lse + static_cast<size_t>(row) * a.hf + h) * kLog2e;
  }

  // Row-pass epilogue: dq = scale (A - D^ B) / L in the feature dtype, and the record
  // (lse2 + log2 L, D^) with D^ = D / L (one lane per head writes it).
  __device__ __forceinline__ static void finish_row(const BwdArgs& a, int row, int r, int h,
                                                    float lse2, const float* A, const float* Bk,
                                                    float D, float Lp) {
    const float inv = Lp > 0.f ? 1.f / Lp : 0.f;
    const float Dn = D * inv;
    float x[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) x[c] = fmaf(-Dn, Bk[c], A[c]);
    store(a.dq, row, r, x, a.scale * inv, a.ld);
    if (r % LH == 0)
      st_stream(reinterpret_cast<f32x2*>(a.ws_ld) + static_cast<size_t>(row) * a.hf + h,
                f32x2{Lp > 0.f ? lse2 + __log2f(Lp) : lse2, Dn});
  }

};

// dQ pass. Hub-row chunk partial layout in ws_dq (full row of F_full elements and H_full
// heads): [chunk][A: F_full | B: F_full | D: H_full | L: H_full, padded to 4] fp32
// (a.dq_stride floats per chunk, a multiple of 4 so the 16-byte stores stay aligned). The
// main kernel works on a feature slice of G lanes (whole heads; see fwd_main); each slice
// writes its part of A, B, D and L.
template <typename T, int G, int LH, int U, int UL>
__global__ __launch_bounds__(kBlock) GA_OCCUPANCY void bwd_dq_main(BwdArgs a0) {
  using K = Bwd<T, G, LH, U>;
  using KL = Bwd<T, G, LH, UL>;  // light rows
  using raw_t = typename K::raw_t;
  constexpr int NG = K::NG, VEC = K::VEC, H = K::H;
  const int lane = threadIdx.x & (kWave - 1);
  const SliceItem si = slice_of(a0.slices);
  const int item = si.item;
  const int so = si.slice * G, ho = si.slice * H;  // lanes / heads before this slice
  BwdArgs a = a0;
  a.q = static_cast<const raw_t*>(a0.q) + so;
  a.k = static_cast<const raw_t*>(a0.k) + so;
  a.v = static_cast<const raw_t*>(a0.v) + so;
  a.dout = static_cast<const raw_t*>(a0.dout) + so;
  a.dq = static_cast<raw_t*>(a0.dq) + so;
  a.lse = a0.lse + ho;
  a.ws_ld = a0.ws_ld + 2 * ho;
  const int g = lane / G, r = lane % G, h = r / LH;
  const DevBins& B = a.rows;
  typename K::raw_t qr, dor;
  float A[VEC], Bk[VEC], lse2, D = 0.f, Lp = 0.f;
#pragma unroll
  for (int c = 0; c < VEC; ++c) A[c] = Bk[c] = 0.f;
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
    K::row_prologue(a, row, r, h, qr, dor, lse2);
    K::template run_dq<NG>(a, e0, e1, 0, g, r, qr, dor, lse2, A, Bk, D, Lp);
    K::template group_sum<NG>(A);
    K::template group_sum<NG>(Bk);
    K::template group_sum1<NG>(D);
    K::template group_sum1<NG>(Lp);
    if (g != 0) return;
    if (chunk) {
      const int Ff = a.ld * VEC;  // elements of the full row
      float* p = a.ws_dq + static_cast<size_t>(c) * a.dq_stride;
      K::store_f32(p + so * VEC, r, A);
      K::store_f32(p + Ff + so * VEC, r, Bk);
      if (r % LH == 0) {
        st_stream(p + 2 * Ff + ho + h, D);
        st_stream(p + 2 * Ff + a.hf + ho + h, Lp);
      }
    } else {
      K::finish_row(a, row, r, h, lse2, A, Bk, D, Lp);
    }
    return;
  }
  const int li = (item - B.n_sched - B.n_medium) * NG + g;
  if (li >= B.n_light) return;
  const int row = B.light[li];
  const int e0 = a.indptr[row], e1 = a.indptr[row + 1];
  K::row_prologue(a, row, r, h, qr, dor, lse2);
  KL::template run_dq<1>(a, e0, e1, g * G, 0, r, qr, dor, lse2, A, Bk, D, Lp);
  K::finish_row(a, row, r, h, lse2, A, Bk, D, Lp);
}

// One wavefront per hub row: lane group g sums chunks c0+g, c0+g+NG, ... in ascending
// order, then the group sums are added by the fixed butterfly (deterministic).
template <typename T, int G, int LH>
__global__ __launch_bounds__(kBlock) void bwd_dq_merge(BwdArgs a) {
  using K = Bwd<T, G, LH, 1>;
  constexpr int VEC = K::VEC, F = K::F, H = K::H, NG = K::NG;
  const int hub = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane / G, r = lane % G, h = r / LH;
  if (hub >= a.rows.n_hub) return;
  const int row = a.rows.hub[hub];
  const int c0 = a.rows.hub_chunk_ptr[hub], c1 = a.rows.hub_chunk_ptr[hub + 1];
  float A[VEC], Bk[VEC], D = 0.f, Lp = 0.f;
#pragma unroll
  for (int c = 0; c < VEC; ++c) A[c] = Bk[c] = 0.f;
#pragma unroll 4
  for (int c = c0 + g; c < c1; c += NG) {
    const float* p = a.ws_dq + static_cast<size_t>(c) * a.dq_stride;
    K::add_f32(p, r, A);
    K::add_f32(p + F, r, Bk);
    D += ld_stream(p + 2 * F + h);
    Lp += ld_stream(p + 2 * F + H + h);
  }
  K::template group_sum<NG>(A);
  K::template group_sum<NG>(Bk);
  K::template group_sum1<NG>(D);
  K::template group_sum1<NG>(Lp);
  if (g != 0) return;
  const float lse2 = ld_stream(a.lse + static_cast<size_t>(row) * a.hf + h) * kLog2e;
  K::finish_row(a, row, r, h, lse2, A, Bk, D, Lp);
}

template <typename T, int G, int LH, int U, int UL>
__global__ __launch_bounds__(kBlock) GA_OCCUPANCY void bwd_dkdv_main(BwdArgs a) {
  using K = Bwd<T, G, LH, U>;
  using KL = Bwd<T, G, LH, UL>;  // light columns
  constexpr int NG = K::NG, VEC = K::VEC, F = K::F;
  const int lane = threadIdx.x & (kWave - 1);
  const int item = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int g = lane / G, r = lane % G, h = r / LH;
  const DevBins& B = a.cols;
  typename K::raw_t kr, vr;
  typename K::acc_t dk[VEC], dv[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) dk[c] = dv[c] = 0;
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
    const size_t off = static_cast<size_t>(col) * G + r;
    kr = ld_stream(K::R(a.k) + off);
    vr = ld_stream(K::R(a.v) + off);
    K::template run_dkdv<NG>(a, e0, e1, 0, g, r, h, kr, vr, dk, dv);
    K::template group_sum<NG>(dk);
    K::template group_sum<NG>(dv);
    if (g != 0) return;
    if (chunk) {
      float* p = a.ws_dkv + static_cast<size_t>(c) * 2 * F;
      K::store_f32(p, r, dk);
      K::store_f32(p + F, r, dv);
    } else {
      K::store(a.dk, col, r, dk, a.scale);
      K::store(a.dv, col, r, dv, 1.f);
    }
    return;
  }
  const int li = (item - B.n_sched - B.n_medium) * NG + g;
  if (li >= B.n_light) return;
  const int col = B.light[li];
  const int e0 = a.colptr[col], e1 = a.colptr[col + 1];
  const size_t off = static_cast<size_t>(col) * G + r;
  kr = ld_stream(K::R(a.k) + off);
  vr = ld_stream(K::R(a.v) + off);
  KL::template run_dkdv<1>(a, e0, e1, g * G, 0, r, h, kr, vr, dk, dv);
  K::store(a.dk, col, r, dk, a.scale);
  K::store(a.dv, col, r, dv, 1.f);
}

template <typename T, int G, int LH>
__global__ __launch_bounds__(kBlock) void bwd_dkdv_merge(BwdArgs a) {
  using K = Bwd<T, G, LH, 1>;
  constexpr int VEC = K::VEC, F = K::F, NG = K::NG;
  const int hub = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane / G, r = lane % G;
  if (hub >= a.cols.n_hub) return;
  const int col = a.cols.hub[hub];
  const int c0 = a.cols.hub_chunk_ptr[hub], c1 = a.cols.hub_chunk_ptr[hub + 1];
  typename K::acc_t dk[VEC], dv[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) dk[c] = dv[c] = 0;
#pragma unroll 4
  for (int c = c0 + g; c < c1; c += NG) {
    const float* p = a.ws_dkv + static_cast<size_t>(c) * 2 * F;
    K::add_f32(p, r, dk);
    K::add_f32(p + F, r, dv);
  }
  K::template group_sum<NG>(dk);
  K::template group_sum<NG>(dv);
  if (g != 0) return;
  K::store(a.dk, col, r, dk, a.scale);
  K::store(a.dv, col, r, dv, 1.f);
}

template <typename T, int G, int LH>
struct Launcher {
  static constexpr int NG = kWave / G;
  static int64_t items_of(const DevBins& B) {
    return int64_t(B.n_sched) + B.n_medium + (int64_t(B.n_light) + NG - 1) / NG;
  }
  template <typename Kern>
  static int go(const char* name, Kern kernel, int64_t blocks, const BwdArgs& a, void* stream,
                TimerHook hook) {
    if (blocks <= 0) return 0;
    if (hook) hook(name, stream, 1);
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), a);
    if (hook) hook(name, stream, 0);
    return static_cast<int>(hipGetLastError());
  }
  // dQ main pass on the slice geometry (G lanes per slice, a.slices slices)
  static int dq_main(const BwdArgs& a, void* stream, TimerHook hook) {
    const int64_t items = items_of(a.rows);
    if (items <= 0) return 0;
    return go("bwd_dq_main", bwd_dq_main<T, G, LH, GA_UNROLL_DQ, GA_UNROLL_DQ_LIGHT>,
              slice_blocks((items + kWavesPerBlock - 1) / kWavesPerBlock, a.slices), a, stream,
              hook);
  }
  // the rest on the full row geometry
  static int rest(const BwdArgs& a, void* stream, TimerHook hook) {
    int e;
    if ((e = go("bwd_dq_merge", bwd_dq_merge<T, G, LH>,
                (a.rows.n_hub + kWavesPerBlock - 1) / kWavesPerBlock, a, stream, hook)))
      return e;
    if ((e = go("bwd_dkdv_main", bwd_dkdv_main<T, G, LH, GA_UNROLL_DKDV, GA_UNROLL_DKDV_LIGHT>,
                (items_of(a.cols) + kWavesPerBlock - 1) / kWavesPerBlock, a, stream, hook)))
      return e;
    return go("bwd_dkdv_merge", bwd_dkdv_merge<T, G, LH>,
              (a.cols.n_hub + kWavesPerBlock - 1) / kWavesPerBlock, a, stream, hook);
  }
};

#define GA_GEOMS(X)                                                                       \
  X(4, 2) X(4, 4) X(8, 2) X(8, 4) X(8, 8) X(16, 2) X(16, 4) X(16, 8) X(16, 16) X(32, 2) \
  X(32, 4) X(32, 8) X(32, 16) X(32, 32) X(64, 2) X(64, 4) X(64, 8) X(64, 16) X(64, 32) \
  X(64, 64)

template <typename T>
int dispatch(const Geometry& g, const BwdArgs& a, void* stream, TimerHook hook) {
  const int GS = g.G / a.slices;
  int e = -1;
#define GA_CASE(GG, LL) \
  if (GS == GG && g.LH == LL) e = Launcher<T, GG, LL>::dq_main(a, stream, hook);
  GA_GEOMS(GA_CASE)
#undef GA_CASE
  if (e) return e;
#define GA_CASE(GG, LL) \
  if (g.G == GG && g.LH == LL) return Launcher<T, GG, LL>::rest(a, stream, hook);
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

bool bwd_supported(ga_dtype dt, const Geometry& g) {
  return (dt == GA_F32 || dt == GA_BF16) && geom_ok(g);
}

int launch_bwd(ga_dtype dt, const Geometry& g, const BwdArgs& a, int64_t, void* stream,
               TimerHook hook) {
  return dt == GA_F32 ? dispatch<float>(g, a, stream, hook) : dispatch<bf16_t>(g, a, stream, hook);
}

}  // namespace ga
