// Backward kernels of the GAT-style score e_ij = scale * LeakyReLU_a(s_i + t_j) for gfx950.
//
// Method: "On Efficient Scaling of GNNs via IO-Aware Layers Implementations", Technical
// Summary > Methodology, attention-based layers, backward pass (weights recomputed from the
// per-node log-sum-exp; transposed adjacency cached for the backward).
//
// With x_ij = s_i + t_j, g_ij = LeakyReLU'(x_ij) (1 for x >= 0, else a), P_ij =
// exp(e_ij - lse_i), dp_ij = <dout_i, v_j>, D_i = sum_j P_ij dp_ij, dS_ij = P_ij (dp_ij - D_i):
//   bwd_gat_rows_main   over CSR rows, one pass per row and head:
//                       L = sum P, D = sum P dp, A = sum P dp g, B = sum P g; with the
//                       weights renormalised by L (1 up to the stored lse's rounding),
//                       D^ = D / L and ds_i = scale (A - D^ B) / L; the record
//                       (lse_i log2 e + log2 L, D^_i) goes to the column pass
//                       (hub rows: fp32 chunk partials of (A, B, D, L))
//   bwd_gat_rows_merge  hub rows: sum chunk partials in ascending chunk order (strided per
//                       lane group, fixed butterfly)
//   bwd_gat_cols_main   over transpose columns: dt_j = scale sum_i dS_ij g_ij,
//                       dv_j = sum_i P_ij dout_i (hub columns: fp32 chunk partials)
//   bwd_gat_cols_merge  hub columns: ordered sum of partials
// Per edge the row pass gathers t_j (4 bytes per head) and v_j; the column pass gathers
// s_i, dout_i and the (lse, D) record. No atomics; every sum has a fixed order.
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {
namespace {

template <typename T, int G, int LH, int U>
struct BwdGat : RowIO<T, G, LH> {
  using IO = RowIO<T, G, LH>;
  using typename IO::L16;
  using typename IO::raw_t;
  using IO::F;
  using IO::H;
  using IO::NG;
  using IO::R;
  using IO::VEC;
  using typename IO::acc_t;
  // chunk partial strides (floats, multiples of 4 so 16-byte accesses stay aligned)
  static constexpr int kRowStride = (4 * H + 3) / 4 * 4;  // A[H] B[H] D[H] L[H]
  static constexpr int kColStride = F + (H + 3) / 4 * 4;   // dv[F] dt[H]

  __device__ __forceinline__ static float lrelu(float x, float a) { return x >= 0.f ? x : x * a; }
  __device__ __forceinline__ static float lrelu_grad(float x, float a) {
    return x >= 0.f ? 1.f : a;
  }

  // Row pass over edges [e0, e1): accumulates D, A, B, L (per head, replicated over the
  // head's lanes).
  template <int NGS>
  __device__ __forceinline__ static void run_rows(const BwdArgs& a, int e0, int e1, int seg0,
                                                  int gs, int r, int h, float si,
                                                  const raw_t& dor, float lse2, float& A,
                                                  float& Bg, float& D, float& Lp) {
    constexpr int L = NGS * G;
    const int lane = threadIdx.x & (kWave - 1);
    const float* __restrict__ Tt = static_cast<const float*>(a.k);
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
        raw_t vr[U];
        float tv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          tv[u] = Tt[static_cast<size_t>(jj[u]) * H + h];
          vr[u] = Vr[static_cast<size_t>(jj[u]) * G + r];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float x = si + tv[u];
          const float s2 = lrelu(x, a.neg_slope) * a.sc2;
          const float dp = head_sum<LH>(L16::dot(dor, vr[u]));
          const float p = ok[u] ? fast_exp2(s2 - lse2) : 0.f;
          const float pg = p * lrelu_grad(x, a.neg_slope);
          D = fmaf(p, dp, D);
          A = fmaf(pg, dp, A);
          Bg += pg;
          Lp += p;
        }
      }
    }
  }

  // Column pass over transpose edges [e0, e1) of column j (t_j, v_j held by the lane).
  template <int NGS>
  __device__ __forceinline__ static void run_cols(const BwdArgs& a, int e0, int e1, int seg0,
                                                  int gs, int r, int h, float tj,
                                                  const raw_t& vr, acc_t& dt, acc_t* dv) {
    constexpr int L = NGS * G;
    const int lane = threadIdx.x & (kWave - 1);
    const float* __restrict__ Ss = static_cast<const float*>(a.q);
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
        raw_t dr[U];
        float sv[U];
        f32x2 ld[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          sv[u] = Ss[static_cast<size_t>(ii[u]) * H + h];
          dr[u] = Or[static_cast<size_t>(ii[u]) * G + r];
          ld[u] = LD[static_cast<size_t>(ii[u]) * H + h];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float x = sv[u] + tj;
          const float s2 = lrelu(x, a.neg_slope) * a.sc2;
          const float dp = head_sum<LH>(L16::dot(dr[u], vr));
          const float p = ok[u] ? fast_exp2(s2 - ld[u].x) : 0.f;
          const float ds = p * (dp - ld[u].y);
          dt += static_cast<acc_t>(ds * lrelu_grad(x, a.neg_slope));
          float df[VEC];
          L16::unpack(dr[u], df);
#pragma unroll
          for (int c = 0; c < VEC; ++c)
            dv[c] = fma(static_cast<acc_t>(p), static_cast<acc_t>(df[c]), dv[c]);
        }
      }
    }
  }

  __device__ __forceinline__ static void row_prologue(const BwdArgs& a, int row, int r, int h,
                                                      float& si, raw_t& dor, float& lse2) {
    si = ld_stream(static_cast<const float*>(a.q) + static_cast<size_t>(row) * H + h);
    dor = ld_stream(R(a.dout) + static_cast<size_t>(row) * G + r);
    lse2 = ld_stream(a.lse + static_cast<size_t>(row) * H + h) * kLog2e;
  }

  // ds_i = scale (A - D^ B) / L with D^ = D / L, and the (lse + log2 L, D^) record; one
  // lane per head writes.
  __device__ __forceinline__ static void store_row(const BwdArgs& a, int row, int r, int h,
                                                   float lse2, float A, float Bg, float D,
                                                   float Lp) {
    if (r % LH != 0) return;
    const float inv = Lp > 0.f ? 1.f / Lp : 0.f;
    const float Dn = D * inv;
    const size_t o = static_cast<size_t>(row) * H + h;
    st_stream(static_cast<float*>(a.dq) + o, a.scale * inv * fmaf(-Dn, Bg, A));
    st_stream(reinterpret_cast<f32x2*>(a.ws_ld) + o,
              f32x2{Lp > 0.f ? lse2 + __log2f(Lp) : lse2, Dn});
  }

  __device__ __forceinline__ static void store_col(const BwdArgs& a, int col, int r, int h,
                                                   acc_t dt, const acc_t* dv) {
    if (r % LH == 0)
      st_stream(static_cast<float*>(a.dk) + static_cast<size_t>(col) * H + h,
                static_cast<float>(static_cast<acc_t>(a.scale) * dt));
    IO::store(a.dv, col, r, dv, 1.f);
  }
};

template <typename T, int G, int LH, int U>
__global__ __launch_bounds__(kBlock) GA_OCCUPANCY void bwd_gat_rows_main(BwdArgs a) {
  using K = BwdGat<T, G, LH, U>;
  constexpr int NG = K::NG;
  const int lane = threadIdx.x & (kWave - 1);
  const int item = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int g = lane / G, r = lane % G, h = r / LH;
  const DevBins& B = a.rows;
  typename K::raw_t dor;
  float si, lse2, A = 0.f, Bg = 0.f, D = 0.f, Lp = 0.f;
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
    K::row_prologue(a, row, r, h, si, dor, lse2);
    K::template run_rows<NG>(a, e0, e1, 0, g, r, h, si, dor, lse2, A, Bg, D, Lp);
    K::template group_sum1<NG>(A);
    K::template group_sum1<NG>(Bg);
    K::template group_sum1<NG>(D);
    K::template group_sum1<NG>(Lp);
    if (g != 0) return;
    if (chunk) {
      if (r % LH == 0) {
        float* p = a.ws_dq + static_cast<size_t>(c) * K::kRowStride;
        st_stream(p + h, A);
        st_stream(p + K::H + h, Bg);
        st_stream(p + 2 * K::H + h, D);
        st_stream(p + 3 * K::H + h, Lp);
      }
    } else {
      K::store_row(a, row, r, h, lse2, A, Bg, D, Lp);
    }
    return;
  }
  const int li = (item - B.n_sched - B.n_medium) * NG + g;
  if (li >= B.n_light) return;
  const int row = B.light[li];
  const int e0 = a.indptr[row], e1 = a.indptr[row + 1];
  K::row_prologue(a, row, r, h, si, dor, lse2);
  K::template run_rows<1>(a, e0, e1, g * G, 0, r, h, si, dor, lse2, A, Bg, D, Lp);
  K::store_row(a, row, r, h, lse2, A, Bg, D, Lp);
}

template <typename T, int G, int LH>
__global__ __launch_bounds__(kBlock) void bwd_gat_rows_merge(BwdArgs a) {
  using K = BwdGat<T, G, LH, 1>;
  constexpr int H = K::H, NG = K::NG;
  const int hub = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane / G, r = lane % G, h = r / LH;
  if (hub >= a.rows.n_hub) return;
  const int row = a.rows.hub[hub];
  const int c0 = a.rows.hub_chunk_ptr[hub], c1 = a.rows.hub_chunk_ptr[hub + 1];
  float A = 0.f, Bg = 0.f, D = 0.f, Lp = 0.f;
#pragma unroll 4
  for (int c = c0 + g; c < c1; c += NG) {
    const float* p = a.ws_dq + static_cast<size_t>(c) * K::kRowStride;
    A += ld_stream(p + h);
    Bg += ld_stream(p + H + h);
    D += ld_stream(p + 2 * H + h);
    Lp += ld_stream(p + 3 * H + h);
  }
  K::template group_sum1<NG>(A);
  K::template group_sum1<NG>(Bg);
  K::template group_sum1<NG>(D);
  K::template group_sum1<NG>(Lp);
  if (g != 0) return;
  const float lse2 = ld_stream(a.lse + static_cast<size_t>(row) * H + h) * kLog2e;
  K::store_row(a, row, r, h, lse2, A, Bg, D, Lp);
}

template <typename T, int G, int LH, int U>
__global__ __launch_bounds__(kBlock) GA_OCCUPANCY void bwd_gat_cols_main(BwdArgs a) {
  using K = BwdGat<T, G, LH, U>;
  constexpr int NG = K::NG, VEC = K::VEC, H = K::H, F = K::F;
  const int lane = threadIdx.x & (kWave - 1);
  const int item = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int g = lane / G, r = lane % G, h = r / LH;
  const DevBins& B = a.cols;
  typename K::raw_t vr;
  float tj;
  typename K::acc_t dt = 0, dv[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) dv[c] = 0;
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
    tj = ld_stream(static_cast<const float*>(a.k) + static_cast<size_t>(col) * H + h);
    vr = ld_stream(K::R(a.v) + static_cast<size_t>(col) * G + r);
    K::template run_cols<NG>(a, e0, e1, 0, g, r, h, tj, vr, dt, dv);
    K::template group_sum1<NG>(dt);
    K::template group_sum<NG>(dv);
    if (g != 0) return;
    if (chunk) {
      float* p = a.ws_dkv + static_cast<size_t>(c) * K::kColStride;
      K::store_f32(p, r, dv);
      if (r % LH == 0) st_stream(p + F + h, static_cast<float>(dt));
    } else {
      K::store_col(a, col, r, h, dt, dv);
    }
    return;
  }
  const int li = (item - B.n_sched - B.n_medium) * NG + g;
  if (li >= B.n_light) return;
  const int col = B.light[li];
  const int e0 = a.colptr[col], e1 = a.colptr[col + 1];
  tj = ld_stream(static_cast<const float*>(a.k) + static_cast<size_t>(col) * H + h);
  vr = ld_stream(K::R(a.v) + static_cast<size_t>(col) * G + r);
  K::template run_cols<1>(a, e0, e1, g * G, 0, r, h, tj, vr, dt, dv);
  K::store_col(a, col, r, h, dt, dv);
}

template <typename T, int G, int LH>
__global__ __launch_bounds__(kBlock) void bwd_gat_cols_merge(BwdArgs a) {
  using K = BwdGat<T, G, LH, 1>;
  constexpr int VEC = K::VEC, F = K::F, NG = K::NG;
  const int hub = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane / G, r = lane % G, h = r / LH;
  if (hub >= a.cols.n_hub) return;
  const int col = a.cols.hub[hub];
  const int c0 = a.cols.hub_chunk_ptr[hub], c1 = a.cols.hub_chunk_ptr[hub + 1];
  typename K::acc_t dt = 0, dv[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) dv[c] = 0;
#pragma unroll 4
  for (int c = c0 + g; c < c1; c += NG) {
    const float* p = a.ws_dkv + static_cast<size_t>(c) * K::kColStride;
    K::add_f32(p, r, dv);
    dt += ld_stream(p + F + h);
  }
  K::template group_sum1<NG>(dt);
  K::template group_sum<NG>(dv);
  if (g != 0) return;
  K::store_col(a, col, r, h, dt, dv);
}

template <typename T, int G, int LH>
int launch(const BwdArgs& a, void* stream, TimerHook hook) {
  constexpr int NG = kWave / G;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto items_of = [](const DevBins& B) {
    return int64_t(B.n_sched) + B.n_medium + (int64_t(B.n_light) + NG - 1) / NG;
  };
  auto go = [&](const char* name, auto kernel, int64_t blocks) -> int {
    if (blocks <= 0) return 0;
    if (hook) hook(name, stream, 1);
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s, a);
    if (hook) hook(name, stream, 0);
    return static_cast<int>(hipGetLastError());
  };
  int e;
  if ((e = go("bwd_gat_rows_main", bwd_gat_rows_main<T, G, LH, GA_UNROLL_DQ>,
              (items_of(a.rows) + kWavesPerBlock - 1) / kWavesPerBlock)))
    return e;
  if ((e = go("bwd_gat_rows_merge", bwd_gat_rows_merge<T, G, LH>,
              (a.rows.n_hub + kWavesPerBlock - 1) / kWavesPerBlock)))
    return e;
  if ((e = go("bwd_gat_cols_main", bwd_gat_cols_main<T, G, LH, GA_UNROLL_DKDV>,
              (items_of(a.cols) + kWavesPerBlock - 1) / kWavesPerBlock)))
    return e;
  if ((e = go("bwd_gat_cols_merge", bwd_gat_cols_merge<T, G, LH>,
              (a.cols.n_hub + kWavesPerBlock - 1) / kWavesPerBlock)))
    return e;
  return 0;
}

#define GA_GEOMS(X)                                                                       \
  X(4, 2) X(4, 4) X(8, 2) X(8, 4) X(8, 8) X(16, 2) X(16, 4) X(16, 8) X(16, 16) X(32, 2) \
  X(32, 4) X(32, 8) X(32, 16) X(32, 32) X(64, 2) X(64, 4) X(64, 8) X(64, 16) X(64, 32) \
  X(64, 64)

template <typename T>
int dispatch(const Geometry& g, const BwdArgs& a, void* stream, TimerHook hook) {
#define GA_CASE(GG, LL) \
  if (g.G == GG && g.LH == LL) return launch<T, GG, LL>(a, stream, hook);
  GA_GEOMS(GA_CASE)
#undef GA_CASE
  return -1;
}

}  // namespace

int launch_bwd_gat(ga_dtype dt, const Geometry& g, const BwdArgs& a, void* stream,
                   TimerHook hook) {
  return dt == GA_F32 ? dispatch<float>(g, a, stream, hook) : dispatch<bf16_t>(g, a, stream, hook);
}

}  // namespace ga
