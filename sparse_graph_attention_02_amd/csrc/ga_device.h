// Device helpers for the gfx950 (CDNA4) kernels: 16-byte lane vectors, bf16 conversion,
// cross-lane sums within a head (DPP / ds_swizzle), work-item decoding.
//
// Lane layout used by every kernel: a feature row of H*d elements is split into G lanes
// of 16 bytes each (lane r holds elements [r*VEC, (r+1)*VEC)); a head spans LH = G/H
// consecutive lanes. A 64-lane wavefront holds NG = 64/G such lane groups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ga_internal.h"

namespace ga {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running maximum of an empty state: finite, so exp2(m_old - m_new) never sees inf - inf.
constexpr float kEmptyMax = -1.0e30f;

// bf16 is carried as raw 16-bit patterns.
using bf16_t = uint16_t;

// 16-byte lane vectors as clang ext-vector types (accepted by the non-temporal builtins).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Loads/stores of data a pass touches exactly once (index batches, the row-side operand,
// outputs, partials) carry the non-temporal hint so they do not evict the gathered
// neighbour rows, which power-law graphs re-read from L2.
template <typename V>
__device__ __forceinline__ V ld_stream(const V* p) {
  return __builtin_nontemporal_load(p);
}
template <typename V>
__device__ __forceinline__ void st_stream(V* p, V x) {
  __builtin_nontemporal_store(x, p);
}

// Gathered neighbour rows are read through a structured buffer: one descriptor per tensor
// (base, row stride in bytes, number of rows), and each load names a node id and this lane's
// byte offset within the row. The memory unit forms the address (id * stride + offset, a
// 32-bit byte offset from the base), so no address arithmetic runs on the vector ALU, and an
// id outside [0, rows) reads zeros. A table larger than 4 GiB does not fit one descriptor;
// kernels read those with plain 64-bit loads (ld_node below, `wide`). The fourth
// descriptor word selects 32-bit untyped data (the gfx9 buffer format).
constexpr int kBufWord3 = 0x00020000;
using rows_t = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ rows_t node_rows(const void* base, int row_bytes, int n_rows) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base),
                                           static_cast<short>(row_bytes), n_rows, kBufWord3);
}
__device__ u32x4 ga_sbuf_ld_v4(rows_t rows, int index, int offset, int soffset, int aux)
    __asm("llvm.amdgcn.struct.ptr.buffer.load.v4i32");
__device__ float ga_sbuf_ld_f32(rows_t rows, int index, int offset, int soffset, int aux)
    __asm("llvm.amdgcn.struct.ptr.buffer.load.f32");
template <typename V>
__device__ __forceinline__ V ld_row(rows_t rows, int node, int offset) {
  if constexpr (sizeof(V) == 16) {
    return __builtin_bit_cast(V, ga_sbuf_ld_v4(rows, node, offset, 0, 0));
  } else {
    static_assert(sizeof(V) == 4, "16- or 4-byte row elements");
    return __builtin_bit_cast(V, ga_sbuf_ld_f32(rows, node, offset, 0, 0));
  }
}
// Element r (16-byte lanes) of row `node` of a table with rows of ld lanes: through the
// descriptor, or (WIDE: a table past 4 GiB) by a plain load. WIDE is a kernel template
// parameter, or a uniform branch taken once per step around a step's loads.
template <bool WIDE, typename V>
__device__ __forceinline__ V ld_node(rows_t rows, const V* base, int node, int ld, int r) {
  if constexpr (WIDE)
    return base[static_cast<size_t>(static_cast<uint32_t>(node)) * ld + r];
  else
    return ld_row<V>(rows, node, r * int(sizeof(V)));
}

// Edges folded per lane group per step (independent gathers in flight per lane), per pass.
#ifndef GA_UNROLL_FWD
#define GA_UNROLL_FWD 8
#endif
#ifndef GA_UNROLL_DQ
#define GA_UNROLL_DQ 4
#endif
#ifndef GA_UNROLL_DKDV
#define GA_UNROLL_DKDV 4
#endif
// The same for light rows and columns (at most light_max_deg edges, on power-law graphs
// mostly a few): fewer slots per step, as masked slots still pay for the score and the
// exponential.
#ifndef GA_UNROLL_FWD_LIGHT
#define GA_UNROLL_FWD_LIGHT 2
#endif
#ifndef GA_UNROLL_DQ_LIGHT
#define GA_UNROLL_DQ_LIGHT 4
#endif
#ifndef GA_UNROLL_DKDV_LIGHT
#define GA_UNROLL_DKDV_LIGHT 4
#endif
// Minimum waves per SIMD requested from the register allocator for the main kernels
// (0 = compiler default).
#ifndef GA_WAVES_PER_EU
#define GA_WAVES_PER_EU 0
#endif
#if GA_WAVES_PER_EU > 0
#define GA_OCCUPANCY __attribute__((amdgpu_waves_per_eu(GA_WAVES_PER_EU)))
#else
#define GA_OCCUPANCY
#endif

template <typename T>
struct Lane16;

template <>
struct Lane16<float> {
  using raw_t = f32x4;
  static constexpr int VEC = 4;
  __device__ __forceinline__ static void unpack(const raw_t& x, float* f) {
    f[0] = x.x;
    f[1] = x.y;
    f[2] = x.z;
    f[3] = x.w;
  }
  __device__ __forceinline__ static raw_t pack(const float* f) {
    return raw_t{f[0], f[1], f[2], f[3]};
  }
  // <x, y> over the lane's 4 elements, fp32 FMA chain.
  __device__ __forceinline__ static float dot(const raw_t& x, const raw_t& y) {
    return fmaf(x.w, y.w, fmaf(x.z, y.z, fmaf(x.y, y.y, x.x * y.x)));
  }
  __device__ __forceinline__ static float dot_packed(const raw_t& x, const raw_t& y) {
    return dot(x, y);
  }
};

// fp32 -> bf16 by round-to-nearest-even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

template <>
struct Lane16<bf16_t> {
  using raw_t = u32x4;
  static constexpr int VEC = 8;
  __device__ __forceinline__ static void unpack(const raw_t& x, float* f) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f[2 * c] = __uint_as_float(w[c] << 16);
      f[2 * c + 1] = __uint_as_float(w[c] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static raw_t pack(const float* f) {
    uint32_t w[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = bf16_rne(f[2 * c]) | (bf16_rne(f[2 * c + 1]) << 16);
    return raw_t{w[0], w[1], w[2], w[3]};
  }
  // <x, y> over the lane's 8 bf16 elements (unpack + fp32 FMA chain; a v_dot2_f32_bf16
  // chain measured slower on gfx950 for these gather-bound passes).
  __device__ __forceinline__ static float dot(const raw_t& x, const raw_t& y) {
    float a[8], b[8];
    unpack(x, a);
    unpack(y, b);
    float d = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) d = fmaf(a[c], b[c], d);
    return d;
  }
  // The same sum by four v_dot2_f32_bf16 (two exact bf16 products per instruction, fp32
  // accumulation): half the instructions, for passes bound by VALU issue.
  __device__ __forceinline__ static float dot_packed(const raw_t& x, const raw_t& y) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const uint32_t wx[4] = {x.x, x.y, x.z, x.w}, wy[4] = {y.x, y.y, y.z, y.w};
    float d = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bf16x2_t p, q;
      __builtin_memcpy(&p, &wx[k], 4);
      __builtin_memcpy(&q, &wy[k], 4);
      d = __builtin_amdgcn_fdot2_f32_bf16(p, q, d, false);
    }
    return d;
  }
};

// DPP move within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over the LH consecutive lanes of a head (LH a power of two, head-aligned); every
// lane of the head receives the sum. The summation tree is fixed, so results are
// deterministic.
template <int LH>
__device__ __forceinline__ float head_sum(float x) {
  static_assert(LH >= 1 && LH <= 64 && (LH & (LH - 1)) == 0, "LH must be a power of two");
  if constexpr (LH >= 2) x += dpp_mov<0xb1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (LH >= 4) x += dpp_mov<0x4e>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (LH >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror: other quad of 8
  if constexpr (LH >= 16) x += dpp_mov<0x140>(x); // row_mirror: other half of 16
  if constexpr (LH >= 32)                          // lane ^ 16 within 32 (bitmask swizzle)
    x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401f));
  if constexpr (LH >= 64) x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row-slice I/O shared by the backward kernels: a lane owns VEC elements of a feature row
// (G lanes per row, LH lanes per head, NG lane groups per wavefront).
template <typename T, int G, int LH>
struct RowIO {
  using L16 = Lane16<T>;
  using raw_t = typename L16::raw_t;
  static constexpr int VEC = L16::VEC;
  static constexpr int NG = kWave / G;
  static constexpr int H = G / LH;
  static constexpr int F = G * VEC;
  // Accumulator of the column-pass sums (dK, dV, dt). A source column's weights are not
  // normalised and its sum can cancel heavily (thousands of terms for a hub column), so
  // fp32 features accumulate in fp64 to keep fp32-level accuracy in the result; bf16
  // features keep fp32 accumulation.
  using acc_t = std::conditional_t<std::is_same_v<T, float>, double, float>;

  __device__ __forceinline__ static const raw_t* R(const void* p) {
    return static_cast<const raw_t*>(p);
  }
  // x * mul, converted to T, into row `row` of a [N, H*d] array (streamed store); ld = the
  // row stride in 16-byte lanes (G unless the kernel works on a slice of a wider row).
  template <typename X>
  __device__ __forceinline__ static void store(void* base, int row, int r, const X* x,
                                               float mul, int ld = G) {
    float o[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) o[c] = static_cast<float>(x[c] * static_cast<X>(mul));
    st_stream(static_cast<raw_t*>(base) + static_cast<size_t>(row) * ld + r, L16::pack(o));
  }
  // fp32 row-slice store / accumulate (chunk partials are fp32; X is the accumulator).
  template <typename X>
  __device__ __forceinline__ static void store_f32(float* base, int r, const X* x) {
    f32x4* p = reinterpret_cast<f32x4*>(base + r * VEC);
#pragma unroll
    for (int c = 0; c < VEC / 4; ++c)
      st_stream(p + c, f32x4{static_cast<float>(x[4 * c]), static_cast<float>(x[4 * c + 1]),
                             static_cast<float>(x[4 * c + 2]), static_cast<float>(x[4 * c + 3])});
  }
  template <typename X>
  __device__ __forceinline__ static void add_f32(const float* base, int r, X* x) {
    const f32x4* p = reinterpret_cast<const f32x4*>(base + r * VEC);
#pragma unroll
    for (int c = 0; c < VEC / 4; ++c) {
      const f32x4 y = ld_stream(p + c);
      x[4 * c] += y.x;
      x[4 * c + 1] += y.y;
      x[4 * c + 2] += y.z;
      x[4 * c + 3] += y.w;
    }
  }
  // Sums over the NGS lane groups of a segment (butterfly over lane distance G, fixed order).
  template <int NGS, typename X>
  __device__ __forceinline__ static void group_sum(X* x) {
#pragma unroll
    for (int off = G; off < NGS * G; off <<= 1)
#pragma unroll
      for (int c = 0; c < VEC; ++c) x[c] += __shfl_xor(x[c], off);
  }
  template <int NGS, typename X>
  __device__ __forceinline__ static void group_sum1(X& x) {
#pragma unroll
    for (int off = G; off < NGS * G; off <<= 1) x += __shfl_xor(x, off);
  }
};

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Feature slices dealt to XCDs. The hardware hands workgroups to the 8 XCDs round-robin by
// block id, and each XCD has its own L2. A launch whose work items are split into S feature
// slices (S dividing 8) maps block b to slice (b mod 8) / (8 / S): every XCD then caches
// only its slice of the gathered rows, so hot source rows take S times less of its L2 and
// are re-read S times as often there. Returns the wave's slice and its work item within
// the slice; the grid is slice_blocks(blocks per slice, S) blocks, and items past the
// slice's end are the caller's to skip. S = 1 is the plain mapping.
struct SliceItem {
  int slice, item;
};
__device__ __forceinline__ SliceItem slice_of(int S) {
  const int wave = threadIdx.x >> 6;
  if (S == 1) return {0, wave_uniform(blockIdx.x * kWavesPerBlock + wave)};
  const int q = 8 / S;  // XCDs per slice
  const int x = blockIdx.x & 7;
  const int blk = (blockIdx.x >> 3) * q + x % q;
  return {wave_uniform(x / q), wave_uniform(blk * kWavesPerBlock + wave)};
}
// Chunk run by chunk slot `slot` (< B.n_sched): the plan's XCD schedule when it has one
// (-1 marks an unused slot), else the chunk of the same index.
__device__ __forceinline__ int chunk_of(const DevBins& B, int slot) {
  return B.sched ? wave_uniform(B.sched[slot]) : slot;
}
static_assert(kWavesPerBlock == kWavesPerSlotBlock, "chunk schedules assume 4-wave blocks");

inline int64_t slice_blocks(int64_t blocks_per_slice, int S) {
  if (S == 1) return blocks_per_slice;
  const int q = 8 / S;
  return 8 * ((blocks_per_slice + q - 1) / q);
}

}  // namespace ga
