// Backward kernels of the GATv2 score for gfx950:
//   e_ij = scale * sum_c a[c] LeakyReLU(z_ij[c]),  z_ij = xd_i + xs_j,  message xs_j.
//
// Method: "On Efficient Scaling of GNNs via IO-Aware Layers Implementations", Technical
// Summary > Methodology, attention-based layers, backward pass (weights recomputed from the
// per-node log-sum-exp; cached transposed adjacency for the backward). GATv2 is the layer
// the pages name; its score is the textbook one.
//
// With g = LeakyReLU'(z) (elementwise), P_ij = exp(e_ij - lse_i), dp_ij = <dout_i, xs_j>,
// L_i = sum_j P_ij (1 up to the stored lse's rounding; the weights are renormalised by it),
// D^_i = sum_j P_ij dp_ij / L_i, dS_ij = P_ij / L_i (dp_ij - D^_i),
//   R_i = sum_j dS_ij g_ij  and  C_j = sum_i dS_ij g_ij  (elementwise):
//   dxd_i = scale a R_i,   dxs_j = scale a C_j + sum_i P_ij dout_i,
//   dattn = scale sum_ij dS_ij LeakyReLU(z_ij) = scale (sum_i xd_i R_i + sum_j xs_j C_j),
// the last because LeakyReLU(z) = g z and z_ij = xd_i + xs_j: the attention gradient costs
// one product per node instead of two per edge.
//   bwd_gatv2_rows_main   over CSR rows (xs rows by structured buffer loads, or plain 64-bit
//                         loads for tables past 4 GiB): per lane element A1 = sum P dp g,
//                         B1 = sum P g, R_i = (A1 - D^ B1) / L; writes dxd, the record
//                         (lse_i log2 e + log2 L_i, D^_i) for the column pass, and
//                         scale xd_i R_i into the wave's dattn partial. Each of the W
//                         wavefronts runs kItemsPerWave work items dealt in snake order (pass
//                         k takes item k W + w, or k W + W-1-w on odd passes; items are sorted
//                         by size, so every wave gets a mix) and writes one fp32 partial
//   bwd_gatv2_rows_merge  hub rows: ordered sums of the chunk partials, then as above (one
//                         partial per hub row)
//   bwd_gatv2_cols_main   over transpose columns, dealt to waves the same way (fewer items
//                         per wave): dxs_j, and scale xs_j C_j into the wave's LDS tile; the
//                         block's four tiles are summed into one partial per block
//   bwd_gatv2_cols_merge  hub columns: ordered sums of partials, then as above
//   bwd_gatv2_da_reduce   fixed-order fp64 tree over all dattn partials (32 rows per block
//                         per stage, ping-pong buffers) -> dattn [H*d]
// No atomics; every sum has a fixed order, so results are bitwise reproducible.
#include "ga_device.h"
#include "ga_internal.h"

namespace ga {
namespace {

constexpr int kItemsPerWave = 16;  // row-pass work items per wavefront (bounds da partials)
// Column-pass work items per wavefront. Fewer than the row pass: the column pass is
// memory-bound and balances best with fine-grained waves; its partials are per block.
#ifndef GA_GV2_COL_ITEMS
#define GA_GV2_COL_ITEMS 4
#endif
constexpr int kColItemsPerWave = GA_GV2_COL_ITEMS;
// Column-pass waves W for `items` work items. With an XCD schedule W is a multiple of
// kXcds * kWavesPerBlock, so that item k W + w runs on the XCD of slot w, the XCD its
// scheduled chunk belongs to; the snake order's mirror then reverses whole groups of that
// many waves, which keeps every wave's XCD.
__host__ __device__ inline int64_t gv2_col_waves(int64_t items, bool sched) {
  constexpr int64_t q = kXcds * kWavesPerBlock;
  const int64_t w = (items + kColItemsPerWave - 1) / kColItemsPerWave;
  return sched ? (w + q - 1) / q * q : w;
}
__host__ __device__ inline int64_t gv2_col_mirror(int64_t w, int64_t W, bool sched) {
  constexpr int64_t q = kXcds * kWavesPerBlock;
  return sched ? (W / q - 1 - w / q) * q + w % q : W - 1 - w;
}
constexpr int kReduceFan = 32;     // rows summed per block in each da reduction stage
// Edges in flight per lane group in the row pass, as many as keep the kernel within 128
// VGPRs (4 waves per SIMD) without spills: 5 for rows of at most 32 lanes with heads of at
// most 4 lanes, 3 for wider rows or heads.
template <int G, int LH>
constexpr int rows_unroll() {
  return (G <= 32 && LH <= 4) ? 5 : 3;
}

template <typename T, int G, int LH, int U>
struct BwdV2 : RowIO<T, G, LH> {
  using IO = RowIO<T, G, LH>;
  using typename IO::L16;
  using typename IO::raw_t;
  using IO::F;
  using IO::H;
  using IO::NG;
  using IO::R;
  using IO::VEC;
  using typename IO::acc_t;
  static constexpr int kRowStride = 2 * F + (2 * H + 3) / 4 * 4;  // A1 B1 [F], D L [H]
  static constexpr int kColStride = 2 * F;                        // C1 C2 [F]

  // A1, B1, D, L feed dxd and, through R_i, dattn: a sum over the whole graph of per-row
  // terms that cancel; for fp32 features they are kept in fp64 (acc_t) so that sum keeps
  // fp32-level accuracy.
  struct RowAcc {
    acc_t A1[VEC], B1[VEC];
    acc_t D, L;
  };

  __device__ __forceinline__ static void zero(RowAcc& s) {
#pragma unroll
    for (int c = 0; c < VEC; ++c) s.A1[c] = s.B1[c] = 0;
    s.D = s.L = 0;
  }

  __device__ __forceinline__ static void load_attn(const BwdArgs& a, int r, float* av) {
    const f32x4* ap = reinterpret_cast<const f32x4*>(a.attn + r * VEC);
#pragma unroll
    for (int k = 0; k < VEC / 4; ++k) {
      const f32x4 x = ap[k];
      av[4 * k] = x.x;
      av[4 * k + 1] = x.y;
      av[4 * k + 2] = x.z;
      av[4 * k + 3] = x.w;
    }
  }

  // e in log2 units of edge (xd, xs): head-summed a . LeakyReLU(xd + xs) * sc2.
  __device__ __forceinline__ static float score2(const BwdArgs& a, const float* xd,
                                                 const float* xs, const float* av) {
    float e = 0.f;
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      const float z = xd[c] + xs[c];
      e = fmaf(av[c], z >= 0.f ? z : z * a.neg_slope, e);
    }
    return head_sum<LH>(e) * a.sc2;
  }

  // Row pass over edges [e0, e1) of a row (xd, dout held by the lane). WIDE: the xs table
  // is larger than one 4 GiB buffer window (BwdArgs::wide).
  template <int NGS, bool WIDE>
  __device__ __forceinline__ static void run_rows(const BwdArgs& a, int e0, int e1, int seg0,
                                                  int gs, int r, const float* xd,
                                                  const raw_t& dor, const float* av,
                                                  float lse2, RowAcc& s) {
    // index batches of whole steps, so that no step of a full batch is part empty (every
    // slot costs its arithmetic here); a step longer than the segment keeps the segment
    constexpr int L = NGS * G, S = NGS * U;
    constexpr int LB = S <= L ? L / S * S : L;
    static_assert(LB > 0 && LB <= L, "index batch");
    const int lane = threadIdx.x & (kWave - 1);
    const rows_t Xd = node_rows(a.k, G * int(sizeof(raw_t)), a.n);
    const raw_t* __restrict__ Xs = R(a.k);
    for (int base = e0; base < e1; base += LB) {
      const int nb = min(LB, e1 - base);
      const int li = lane - seg0;
      // lanes past the batch's edges name node n, one past the table: a structured buffer
      // load out of range returns zeros without touching memory. A step's spare slots read
      // those lanes or, where a step is longer than a batch, lanes of the same batch (edges
      // of this row, weighted zero), so what a table holds outside this row's neighbours
      // never enters the sums. Plain 64-bit loads have no range check; there the spare
      // lanes name the batch's first edge, a neighbour of the same row.
      const int my_j = WIDE ? ld_stream(a.indices + base + (li < nb ? li : 0))
                            : (li < nb ? ld_stream(a.indices + base + li) : a.n);
      // full steps take every slot unmasked; the item's last, partial step skips the slots
      // no lane group of the segment uses (their loads read nothing)
      auto step = [&](int t, auto full) {
        constexpr bool FULL = decltype(full)::value;
        int jj[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int pos = t + u * NGS + gs;
          ok[u] = FULL || pos < nb;
          // a step longer than a lane group's own segment (light rows of 4-lane groups)
          // wraps within that segment, not into the next group's row
          const int src = (S > L && L < kWave) ? (pos & (L - 1)) : pos;
          jj[u] = __builtin_amdgcn_ds_bpermute((seg0 + src) << 2, my_j);
        }
        raw_t xr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) xr[u] = ld_node<WIDE>(Xd, Xs, jj[u], G, r);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if constexpr (!FULL) {
            if (t + u * NGS >= nb) continue;
          }
          float xs[VEC];
          L16::unpack(xr[u], xs);
          // g = LeakyReLU'(z) by one select, LeakyReLU(z) = z g exactly (g is 1 or the slope)
          float g[VEC], e = 0.f;
#pragma unroll
          for (int c = 0; c < VEC; ++c) {
            const float z = xd[c] + xs[c];
            g[c] = z >= 0.f ? 1.f : a.neg_slope;
            e = fmaf(av[c], z * g[c], e);
          }
          const float s2 = head_sum<LH>(e) * a.sc2;
          const float dp = head_sum<LH>(L16::dot_packed(dor, xr[u]));
          const float p = ok[u] ? fast_exp2(s2 - lse2) : 0.f;
          const float pdp = p * dp;
          s.D += static_cast<acc_t>(pdp);
          s.L += static_cast<acc_t>(p);
#pragma unroll
          for (int c = 0; c < VEC; ++c) {
            s.A1[c] = fma(static_cast<acc_t>(pdp), static_cast<acc_t>(g[c]), s.A1[c]);
            s.B1[c] = fma(static_cast<acc_t>(p), static_cast<acc_t>(g[c]), s.B1[c]);
          }
        }
      };
      int t = 0;
      for (; t + S <= nb; t += S) step(t, std::true_type{});
      if (t < nb) step(t, std::false_type{});
    }
  }

  template <int NGS>
  __device__ __forceinline__ static void combine(RowAcc& s) {
    IO::template group_sum<NGS>(s.A1);
    IO::template group_sum<NGS>(s.B1);
    IO::template group_sum1<NGS>(s.D);
    IO::template group_sum1<NGS>(s.L);
  }

  // Row epilogue: dxd, the record, and this row's dattn term scale xd R added into `da`.
  __device__ __forceinline__ static void finish_row(const BwdArgs& a, int row, int r, int h,
                                                    float lse2, const float* av,
                                                    const float* xd, const RowAcc& s,
                                                    acc_t* da) {
    const acc_t inv = s.L > 0 ? acc_t(1) / s.L : acc_t(0);
    const acc_t Dn = s.D * inv;
    const acc_t f = static_cast<acc_t>(a.scale) * inv;
    const float Dn32 = static_cast<float>(Dn);
    float x[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      const acc_t rc = s.A1[c] - Dn * s.B1[c];  // L R_i
      x[c] = av[c] * static_cast<float>(rc);
      da[c] += f * rc * static_cast<acc_t>(xd[c]);
    }
    IO::store(a.dq, row, r, x, static_cast<float>(f));
    if (r % LH == 0) {
      const float L32 = static_cast<float>(s.L);
      st_stream(reinterpret_cast<f32x2*>(a.ws_ld) + static_cast<size_t>(row) * H + h,
                f32x2{L32 > 0.f ? lse2 + __log2f(L32) : lse2, Dn32});
    }
  }

  __device__ __forceinline__ static void store_partial(float* p, int r, int h, const RowAcc& s) {
    IO::store_f32(p, r, s.A1);
    IO::store_f32(p + F, r, s.B1);
    if (r % LH == 0) {
      st_stream(p + 2 * F + h, static_cast<float>(s.D));
      st_stream(p + 2 * F + H + h, static_cast<float>(s.L));
    }
  }

  __device__ __forceinline__ static void add_partial(const float* p, int r, int h, RowAcc& s) {
    IO::add_f32(p, r, s.A1);
    IO::add_f32(p + F, r, s.B1);
    s.D += static_cast<acc_t>(ld_stream(p + 2 * F + h));
    s.L += static_cast<acc_t>(ld_stream(p + 2 * F + H + h));
  }

  // Column pass over transpose edges [e0, e1) of column j (xs_j held by the lane).
  template <int NGS>
  __device__ __forceinline__ static void run_cols(const BwdArgs& a, int e0, int e1, int seg0,
                                                  int gs, int r, int h, const raw_t& xsr,
                                                  const float* xs, const float* av, acc_t* C1,
                                                  acc_t* C2) {
    constexpr int L = NGS * G;
    const int lane = threadIdx.x & (kWave - 1);
    const raw_t* __restrict__ Xd = R(a.q);
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
        raw_t xdr[U], dr[U];
        f32x2 ld[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          xdr[u] = Xd[static_cast<size_t>(ii[u]) * G + r];
          dr[u] = Or[static_cast<size_t>(ii[u]) * G + r];
          ld[u] = LD[static_cast<size_t>(ii[u]) * H + h];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float xd[VEC], df[VEC];
          L16::unpack(xdr[u], xd);
          L16::unpack(dr[u], df);
          const float s2 = score2(a, xd, xs, av);
          const float dp = head_sum<LH>(L16::dot(dr[u], xsr));
          const float p = ok[u] ? fast_exp2(s2 - ld[u].x) : 0.f;
          const float ds = p * (dp - ld[u].y);
#pragma unroll
          for (int c = 0; c < VEC; ++c) {
            const float g = xd[c] + xs[c] >= 0.f ? 1.f : a.neg_slope;
            C1[c] += static_cast<acc_t>(ds * g);
            C2[c] = fma(static_cast<acc_t>(p), static_cast<acc_t>(df[c]), C2[c]);
          }
        }
      }
    }
  }

  // dxs_j = scale a C1 + C2.
  __device__ __forceinline__ static void store_col(const BwdArgs& a, int col, int r,
                                                   const float* av, const acc_t* C1,
                                                   const acc_t* C2) {
    acc_t x[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c)
      x[c] = static_cast<acc_t>(a.scale * av[c]) * C1[c] + C2[c];
    IO::store(a.dk, col, r, x, 1.f);
  }

  // The column's dattn term scale xs_j C_j added into `da` (registers, or the lane's
  // column of an LDS tile [VEC][64] when Stride = kWave).
  template <int Stride = 1>
  __device__ __forceinline__ static void add_col_da(const BwdArgs& a, const float* xs,
                                                    const acc_t* C1, acc_t* da) {
#pragma unroll
    for (int c = 0; c < VEC; ++c)
      da[c * Stride] += static_cast<acc_t>(a.scale) * C1[c] * static_cast<acc_t>(xs[c]);
  }
};

template <typename T, int G, int LH, int U, bool WIDE>
__global__ __launch_bounds__(kBlock) GA_OCCUPANCY void bwd_gatv2_rows_main(BwdArgs a) {
  using K = BwdV2<T, G, LH, U>;
  constexpr int NG = K::NG, VEC = K::VEC, F = K::F;
  const int lane = threadIdx.x & (kWave - 1);
  const int slot = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int g = lane / G, r = lane % G, h = r / LH;
  const DevBins& B = a.rows;
  const int64_t n_items = int64_t(B.n_chunks) + B.n_medium + (int64_t(B.n_light) + NG - 1) / NG;
  const int64_t W = (n_items + kItemsPerWave - 1) / kItemsPerWave;  // waves = da slots
  // waves of the last block past the last slot own no partial: leave before writing one
  if (slot >= W) return;
  float av[VEC];
  typename K::acc_t da[VEC];
  K::load_attn(a, r, av);
#pragma unroll
  for (int c = 0; c < VEC; ++c) da[c] = 0;
  for (int k = 0; k < kItemsPerWave; ++k) {
    const int64_t item = int64_t(k) * W + ((k & 1) ? W - 1 - slot : slot);
    if (item >= n_items) continue;
    typename K::RowAcc s;
    K::zero(s);
    float xd[VEC], lse2;
    typename K::raw_t dor;
    if (item < B.n_chunks + B.n_medium) {
      int row, e0, e1;
      const bool chunk = item < B.n_chunks;
      if (chunk) {
        row = B.chunk_row[item];
        e0 = B.chunk_begin[item];
        e1 = B.chunk_end[item];
      } else {
        row = B.medium[item - B.n_chunks];
        e0 = a.indptr[row];
        e1 = a.indptr[row + 1];
      }
      const size_t off = static_cast<size_t>(row) * G + r;
      K::L16::unpack(ld_stream(K::R(a.q) + off), xd);
      dor = ld_stream(K::R(a.dout) + off);
      lse2 = ld_stream(a.lse + static_cast<size_t>(row) * K::H + h) * kLog2e;
      K::template run_rows<NG, WIDE>(a, e0, e1, 0, g, r, xd, dor, av, lse2, s);
      K::template combine<NG>(s);
      if (g == 0) {
        if (chunk)
          K::store_partial(a.ws_dq + static_cast<size_t>(item) * K::kRowStride, r, h, s);
        else
          K::finish_row(a, row, r, h, lse2, av, xd, s, da);
      }
    } else {
      const int64_t li = (item - B.n_chunks - B.n_medium) * NG + g;
      if (li < B.n_light) {
        const int row = B.light[li];
        const int e0 = a.indptr[row], e1 = a.indptr[row + 1];
        const size_t off = static_cast<size_t>(row) * G + r;
        K::L16::unpack(ld_stream(K::R(a.q) + off), xd);
        dor = ld_stream(K::R(a.dout) + off);
        lse2 = ld_stream(a.lse + static_cast<size_t>(row) * K::H + h) * kLog2e;
        K::template run_rows<1, WIDE>(a, e0, e1, g * G, 0, r, xd, dor, av, lse2, s);
        K::finish_row(a, row, r, h, lse2, av, xd, s, da);
      }
    }
  }
  K::template group_sum<NG>(da);
  if (g == 0) K::store_f32(a.ws_da + static_cast<size_t>(slot) * F, r, da);
}

// One wavefront per hub row; its dattn term goes to partial slot slot0 + hub.
template <typename T, int G, int LH>
__global__ __launch_bounds__(kBlock) void bwd_gatv2_rows_merge(BwdArgs a, int64_t slot0) {
  using K = BwdV2<T, G, LH, 1>;
  constexpr int NG = K::NG, VEC = K::VEC, F = K::F, H = K::H;
  const int hub = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane / G, r = lane % G, h = r / LH;
  if (hub >= a.rows.n_hub) return;
  const int row = a.rows.hub[hub];
  const int c0 = a.rows.hub_chunk_ptr[hub], c1 = a.rows.hub_chunk_ptr[hub + 1];
  typename K::RowAcc s;
  K::zero(s);
#pragma unroll 2
  for (int c = c0 + g; c < c1; c += NG)
    K::add_partial(a.ws_dq + static_cast<size_t>(c) * K::kRowStride, r, h, s);
  K::template combine<NG>(s);
  if (g != 0) return;
  float av[VEC], xd[VEC];
  typename K::acc_t da[VEC];
  K::load_attn(a, r, av);
  K::L16::unpack(ld_stream(K::R(a.q) + static_cast<size_t>(row) * G + r), xd);
#pragma unroll
  for (int c = 0; c < VEC; ++c) da[c] = 0;
  const float lse2 = ld_stream(a.lse + static_cast<size_t>(row) * H + h) * kLog2e;
  K::finish_row(a, row, r, h, lse2, av, xd, s, da);
  K::store_f32(a.ws_da + static_cast<size_t>(slot0 + hub) * F, r, da);
}

// One reduction stage: block b sums rows [b*kReduceFan, min((b+1)*kReduceFan, n)) of src
// (row length F) in row order, in fp64, into row b of dst64 (or into dst32 for the last
// stage, which has a single block).
template <typename S>
__global__ __launch_bounds__(kBlock) void bwd_gatv2_da_reduce(const S* __restrict__ src, int64_t n,
                                                              int F, double* __restrict__ dst64,
                                                              float* __restrict__ dst32) {
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * kReduceFan;
  const int64_t s1 = min(n, s0 + kReduceFan);
  for (int c = threadIdx.x; c < F; c += kBlock) {
    double acc = 0.0;
#pragma unroll 8
    for (int64_t sl = s0; sl < s1; ++sl) acc += static_cast<double>(src[sl * F + c]);
    if (dst32)
      dst32[c] = static_cast<float>(acc);
    else
      dst64[static_cast<size_t>(blockIdx.x) * F + c] = acc;
  }
}

// Column pass, dealt like the row pass: wave w of W runs kColItemsPerWave items in snake
// order; block b writes its waves' dattn partial to slot slot0 + b. Chunk items are slots
// of the plan's XCD schedule when it has one (see gv2_col_waves); the row pass runs its
// chunks in chunk order (it is bound by arithmetic, not by L2).
template <typename T, int G, int LH, int U>
__global__ __launch_bounds__(kBlock) GA_OCCUPANCY void bwd_gatv2_cols_main(BwdArgs a,
                                                                       int64_t slot0) {
  using K = BwdV2<T, G, LH, U>;
  constexpr int NG = K::NG, VEC = K::VEC, F = K::F;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int g = lane / G, r = lane % G, h = r / LH;
  const DevBins& B = a.cols;
  const bool sched = B.sched != nullptr;
  const int64_t n_items = int64_t(B.n_sched) + B.n_medium + (int64_t(B.n_light) + NG - 1) / NG;
  const int64_t W = gv2_col_waves(n_items, sched);
  // Each wave's dattn sum lives in LDS, one column of [VEC][64] per lane (touched once per
  // item, so the edge loop keeps its registers); the block's waves are summed at the end
  // into one partial per block.
  __shared__ typename K::acc_t da_lds[kWavesPerBlock][VEC][kWave];
  typename K::acc_t* da = &da_lds[threadIdx.x >> 6][0][lane];
  float av[VEC];
  K::load_attn(a, r, av);
#pragma unroll
  for (int c = 0; c < VEC; ++c) da[c * kWave] = 0;
  // waves of the last block past wave W-1 take no item but still join the block sum
  for (int k = 0; k < kColItemsPerWave && wave < W; ++k) {
    const int64_t item = int64_t(k) * W + ((k & 1) ? gv2_col_mirror(wave, W, sched) : wave);
    if (item >= n_items) continue;
    float xs[VEC];
    typename K::acc_t C1[VEC], C2[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) C1[c] = C2[c] = 0;
    if (item < B.n_sched + B.n_medium) {
      int col, e0, e1, c = 0;
      const bool chunk = item < B.n_sched;
      if (chunk) {
        c = chunk_of(B, static_cast<int>(item));
        if (c < 0) continue;  // unused slot of an XCD schedule
        col = B.chunk_row[c];
        e0 = B.chunk_begin[c];
        e1 = B.chunk_end[c];
      } else {
        col = B.medium[item - B.n_sched];
        e0 = a.colptr[col];
        e1 = a.colptr[col + 1];
      }
      const typename K::raw_t xsr = ld_stream(K::R(a.k) + static_cast<size_t>(col) * G + r);
      K::L16::unpack(xsr, xs);
      K::template run_cols<NG>(a, e0, e1, 0, g, r, h, xsr, xs, av, C1, C2);
      K::template group_sum<NG>(C1);
      K::template group_sum<NG>(C2);
      if (g == 0) {
        if (chunk) {
          float* p = a.ws_dkv + static_cast<size_t>(c) * K::kColStride;
          K::store_f32(p, r, C1);
          K::store_f32(p + F, r, C2);
        } else {
          K::store_col(a, col, r, av, C1, C2);
          K::template add_col_da<kWave>(a, xs, C1, da);
        }
      }
    } else {
      const int64_t li = (item - B.n_sched - B.n_medium) * NG + g;
      if (li < B.n_light) {
        const int col = B.light[li];
        const int e0 = a.colptr[col], e1 = a.colptr[col + 1];
        const typename K::raw_t xsr = ld_stream(K::R(a.k) + static_cast<size_t>(col) * G + r);
        K::L16::unpack(xsr, xs);
        K::template run_cols<1>(a, e0, e1, g * G, 0, r, h, xsr, xs, av, C1, C2);
        K::store_col(a, col, r, av, C1, C2);
        K::template add_col_da<kWave>(a, xs, C1, da);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x >= kWave) return;
  typename K::acc_t dsum[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) {
    dsum[c] = da_lds[0][c][lane];
#pragma unroll
    for (int w = 1; w < kWavesPerBlock; ++w) dsum[c] += da_lds[w][c][lane];
  }
  K::template group_sum<NG>(dsum);
  if (g == 0) K::store_f32(a.ws_da + static_cast<size_t>(slot0 + blockIdx.x) * F, r, dsum);
}

// One wavefront per hub column; its dattn term goes to partial slot slot0 + hub.
template <typename T, int G, int LH>
__global__ __launch_bounds__(kBlock) void bwd_gatv2_cols_merge(BwdArgs a, int64_t slot0) {
  using K = BwdV2<T, G, LH, 1>;
  constexpr int NG = K::NG, VEC = K::VEC, F = K::F;
  const int hub = wave_uniform(blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6));
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane / G, r = lane % G;
  if (hub >= a.cols.n_hub) return;
  const int col = a.cols.hub[hub];
  const int c0 = a.cols.hub_chunk_ptr[hub], c1 = a.cols.hub_chunk_ptr[hub + 1];
  typename K::acc_t C1[VEC], C2[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) C1[c] = C2[c] = 0;
#pragma unroll 4
  for (int c = c0 + g; c < c1; c += NG) {
    const float* p = a.ws_dkv + static_cast<size_t>(c) * K::kColStride;
    K::add_f32(p, r, C1);
    K::add_f32(p + F, r, C2);
  }
  K::template group_sum<NG>(C1);
  K::template group_sum<NG>(C2);
  if (g != 0) return;
  float av[VEC], xs[VEC];
  typename K::acc_t da[VEC];
  K::load_attn(a, r, av);
  K::L16::unpack(ld_stream(K::R(a.k) + static_cast<size_t>(col) * G + r), xs);
#pragma unroll
  for (int c = 0; c < VEC; ++c) da[c] = 0;
  K::store_col(a, col, r, av, C1, C2);
  K::add_col_da(a, xs, C1, da);
  K::store_f32(a.ws_da + static_cast<size_t>(slot0 + hub) * F, r, da);
}

template <typename T, int G, int LH>
int launch(const BwdArgs& a, void* stream, TimerHook hook) {
  constexpr int NG = kWave / G;
  constexpr int F = G * Lane16<T>::VEC;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto waves_of = [](const DevBins& B, int per_wave) {
    const int64_t items = int64_t(B.n_chunks) + B.n_medium + (int64_t(B.n_light) + NG - 1) / NG;
    return (items + per_wave - 1) / per_wave;
  };
  auto blocks = [](int64_t waves) {
    return dim3(static_cast<unsigned>((waves + kWavesPerBlock - 1) / kWavesPerBlock));
  };
  // dattn partial slots: row waves, hub rows, column blocks, hub columns
  const int64_t row_waves = waves_of(a.rows, kItemsPerWave);
  const int64_t col_waves = gv2_col_waves(
      int64_t(a.cols.n_sched) + a.cols.n_medium + (int64_t(a.cols.n_light) + NG - 1) / NG,
      a.cols.sched != nullptr);
  const int64_t col_blocks = (col_waves + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t slot_rh = row_waves, slot_cw = slot_rh + a.rows.n_hub;
  const int64_t slot_ch = slot_cw + col_blocks, n_slots = slot_ch + a.cols.n_hub;
  int e;
  auto done = [&](const char* name) -> int {
    if (hook) hook(name, stream, 0);
    return static_cast<int>(hipGetLastError());
  };
  if (row_waves > 0) {
    if (hook) hook("bwd_gatv2_rows_main", stream, 1);
    if (a.wide)
      hipLaunchKernelGGL((bwd_gatv2_rows_main<T, G, LH, rows_unroll<G, LH>(), true>),
                         blocks(row_waves), dim3(kBlock), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_gatv2_rows_main<T, G, LH, rows_unroll<G, LH>(), false>),
                         blocks(row_waves), dim3(kBlock), 0, s, a);
    if ((e = done("bwd_gatv2_rows_main"))) return e;
  }
  if (a.rows.n_hub > 0) {
    if (hook) hook("bwd_gatv2_rows_merge", stream, 1);
    hipLaunchKernelGGL((bwd_gatv2_rows_merge<T, G, LH>), blocks(a.rows.n_hub), dim3(kBlock), 0,
                       s, a, slot_rh);
    if ((e = done("bwd_gatv2_rows_merge"))) return e;
  }
  if (col_waves > 0) {
    if (hook) hook("bwd_gatv2_cols_main", stream, 1);
    hipLaunchKernelGGL((bwd_gatv2_cols_main<T, G, LH, GA_UNROLL_DKDV>), blocks(col_waves),
                       dim3(kBlock), 0, s, a, slot_cw);
    if ((e = done("bwd_gatv2_cols_main"))) return e;
  }
  if (a.cols.n_hub > 0) {
    if (hook) hook("bwd_gatv2_cols_merge", stream, 1);
    hipLaunchKernelGGL((bwd_gatv2_cols_merge<T, G, LH>), blocks(a.cols.n_hub), dim3(kBlock), 0,
                       s, a, slot_ch);
    if ((e = done("bwd_gatv2_cols_merge"))) return e;
  }
  {
    // fp32 slots -> fp64 rows, then fp64 stages until one block remains; that last stage
    // always runs, so dattn is written even when there are no slots (zeros)
    if (hook) hook("bwd_gatv2_da_reduce", stream, 1);
    double* bufA = a.ws_da64;
    double* bufB = a.ws_da64 + gatv2_reduce_rows_a(n_slots) * F;
    int64_t n = n_slots;
    const double* src64 = nullptr;
    bool first = true;
    while (true) {
      const int64_t nb = (n + kReduceFan - 1) / kReduceFan;
      if (nb <= 1) {
        if (first)
          hipLaunchKernelGGL((bwd_gatv2_da_reduce<float>), dim3(1), dim3(kBlock), 0, s, a.ws_da,
                             n, F, static_cast<double*>(nullptr), a.dattn);
        else
          hipLaunchKernelGGL((bwd_gatv2_da_reduce<double>), dim3(1), dim3(kBlock), 0, s, src64, n,
                             F, static_cast<double*>(nullptr), a.dattn);
        break;
      }
      double* dst = (src64 == bufA) ? bufB : bufA;
      if (first)
        hipLaunchKernelGGL((bwd_gatv2_da_reduce<float>), dim3(static_cast<unsigned>(nb)),
                           dim3(kBlock), 0, s, a.ws_da, n, F, dst, static_cast<float*>(nullptr));
      else
        hipLaunchKernelGGL((bwd_gatv2_da_reduce<double>), dim3(static_cast<unsigned>(nb)),
                           dim3(kBlock), 0, s, src64, n, F, dst, static_cast<float*>(nullptr));
      src64 = dst;
      n = nb;
      first = false;
    }
    if ((e = done("bwd_gatv2_da_reduce"))) return e;
  }
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

int64_t gatv2_da_slots(const ga_plan* p, const Geometry& g) {
  const int64_t NG = kWave / g.G;
  auto waves = [&](const Bins& b, int per_wave) {
    const int64_t items = int64_t(b.chunk_row.size()) + int64_t(b.medium.size()) +
                          (int64_t(b.light.size()) + NG - 1) / NG;
    return (items + per_wave - 1) / per_wave;
  };
  const Bins& c = p->cols;
  const int64_t col_items =
      int64_t(c.sched.empty() ? c.chunk_row.size() : c.sched.size()) + int64_t(c.medium.size()) +
      (int64_t(c.light.size()) + NG - 1) / NG;
  const int64_t col_blocks =
      (gv2_col_waves(col_items, !c.sched.empty()) + kWavesPerBlock - 1) / kWavesPerBlock;
  return waves(p->rows, kItemsPerWave) + int64_t(p->rows.hub.size()) + col_blocks +
         int64_t(p->cols.hub.size());
}

int64_t gatv2_row_partial_floats(int heads, int dim) {
  const int64_t F = int64_t(heads) * dim;
  return 2 * F + (2 * int64_t(heads) + 3) / 4 * 4;
}

// fp64 rows of the two ping-pong buffers of the da reduction: the first stage writes
// ceil(n / fan) rows into buffer A, the second ceil(n / fan^2) into buffer B, and later
// stages alternate within those sizes.
int64_t gatv2_reduce_rows_a(int64_t n_slots) { return (n_slots + kReduceFan - 1) / kReduceFan; }
int64_t gatv2_reduce_rows(int64_t n_slots) {
  const int64_t a = gatv2_reduce_rows_a(n_slots);
  return a + (a + kReduceFan - 1) / kReduceFan;
}

int launch_bwd_gatv2(ga_dtype dt, const Geometry& g, const BwdArgs& a, void* stream,
                     TimerHook hook) {
  return dt == GA_F32 ? dispatch<float>(g, a, stream, hook) : dispatch<bf16_t>(g, a, stream, hook);
}

}  // namespace ga
