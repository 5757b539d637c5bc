// Device helpers for the gfx950 kernels: element types, MFMA fragments,
// ordered score keys and small wave/block reductions.
//
// MFMA fragment layout used by every 16x16 tile here. Lane l of a wave is
// (j = l / 16, n = l % 16). For a 16-row operand tile (16 query rows or 16
// keys of one block), lane (j, n) holds the contiguous chunk
// [j*D/4, (j+1)*D/4) of row n, i.e. D/4 elements = D/2 bytes (bf16) or D
// bytes (fp32), loaded with 16-byte loads. Instruction c of a contraction
// feeds elements [8c, 8c+8) of that chunk (bf16, v_mfma_f32_16x16x32_bf16) or
// element c (fp32, v_mfma_f32_16x16x4_f32). Because both operands use the
// same chunking, the instructions together contract over every d exactly
// once. The 16x16 fp32 result sits in lane (j, n) as rows 4j+i (i = 0..3) of
// column n.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zpd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct BF16 {
  static constexpr int kBytes = 2;
};
struct F32 {
  static constexpr int kBytes = 4;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// One lane's share of a 16-row operand tile: D/4 elements as 16-byte chunks.
template <typename E, int D>
struct Frag {
  static constexpr int kChunks = (D / 4) * E::kBytes / 16;
  u32x4_t v[kChunks];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) v[c] = u32x4_t{0u, 0u, 0u, 0u};
  }
  // p points at the lane's chunk (16-byte aligned).
  __device__ __forceinline__ void load(const void* p) {
    const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int c = 0; c < kChunks; ++c) v[c] = q[c];
  }
  // Sum of squares of the lane's elements, in fp32.
  __device__ __forceinline__ float sumsq() const {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (E::kBytes == 2) {
          const float a = bf16_lo(w[e]), b = bf16_hi(w[e]);
          s = fmaf(a, a, s);
          s = fmaf(b, b, s);
        } else {
          const float a = __uint_as_float(w[e]);
          s = fmaf(a, a, s);
        }
      }
    }
    return s;
  }
};

// acc += A * B^T for two 16-row fragments (A rows = output rows, B rows =
// output columns), contracting over all D elements.
template <typename E, int D>
__device__ __forceinline__ f32x4_t mma_rows(const Frag<E, D>& a,
                                            const Frag<E, D>& b, f32x4_t acc) {
  if constexpr (E::kBytes == 2) {
#pragma unroll
    for (int c = 0; c < Frag<E, D>::kChunks; ++c)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8_t, a.v[c]),
          __builtin_bit_cast(bf16x8_t, b.v[c]), acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int c = 0; c < Frag<E, D>::kChunks; ++c) {
      const uint32_t wa[4] = {a.v[c].x, a.v[c].y, a.v[c].z, a.v[c].w};
      const uint32_t wb[4] = {b.v[c].x, b.v[c].y, b.v[c].z, b.v[c].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(
            __uint_as_float(wa[e]), __uint_as_float(wb[e]), acc, 0, 0, 0);
    }
  }
  return acc;
}

// Order-preserving map of a float score to uint32 (smaller score, smaller
// key); -0 is folded onto +0 so the two compare equal.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float shfl_xor(float v, int m) {
  return __shfl_xor(v, m, 64);
}

// Sum and maximum over each row of 16 lanes, in every lane of the row, on
// the VALU (DPP): lane ^ 1 and lane ^ 2 by quad permutes, then the half-row
// and row mirrors (lane 7 - i within 8, lane 15 - i within 16). Those pair
// the same partial results as lane ^ 4 and lane ^ 8, and every pair is
// added (or maxed) in one order, so the results equal the xor butterfly's
// bit for bit, in all 16 lanes.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  return v;
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}

// v + v(lane ^ 16) and v + v(lane ^ 32) in every lane, on the VALU
// (v_permlane16_swap / v_permlane32_swap exchange 16-lane rows / 32-lane
// halves; with both operands equal, the two results hold the pair).
__device__ __forceinline__ float pairsum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pairsum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Merge two partial softmax statistics (max m, sum z of exp2((x-m)*sl2)).
__device__ __forceinline__ void merge_stats(float& m, float& z, float m2,
                                            float z2, float sl2) {
  const float mn = fmaxf(m, m2);
  const float a = (m == -INFINITY) ? 0.f : z * fast_exp2((m - mn) * sl2);
  const float b = (m2 == -INFINITY) ? 0.f : z2 * fast_exp2((m2 - mn) * sl2);
  m = mn;
  z = a + b;
}

// Block-wide exclusive prefix sum over W waves; returns the exclusive
// prefix of `v` and stores the total in *total. `scratch` holds at least W
// ints of LDS. Contains __syncthreads; every thread must call it.
template <int W>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch,
                                                    int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const int t = scratch[w];
    if (w < wave) before += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

template <int W>
__device__ __forceinline__ int block_min(int v, int* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  int r = scratch[0];
#pragma unroll
  for (int w = 1; w < W; ++w) r = min(r, scratch[w]);
  __syncthreads();
  return r;
}

// Waits for every outstanding memory operation of this wave.
__device__ __forceinline__ void wait_all_memory() {
  __builtin_amdgcn_s_waitcnt(0);
}

}  // namespace zpd
