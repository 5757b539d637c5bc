// Compaction kernel: moves the kept K and V rows of every unit, in order, to
// logical rows [0, k) ([zh] §2.1 re-packing into the first N_max-1 blocks;
// [zh] §2.2 / [de] §2 / [fr] §2.C target blocks when a shared prefix exists).
//
// One workgroup per (unit, K or V). Rows are read through the source table
// and written through the destination table, 16 bytes per lane, so a row of
// 256 bytes is one coalesced 16-lane segment.
//
// In place (n_pinned == 0) the source of row t is keep[t] >= t, and rows
// below the first hole h already hold their own token. The rows [h, k) are
// processed in ascending chunks; every lane finishes all loads of a chunk
// before any lane stores it, so a row is always read before the chunk that
// overwrites it is written (a later chunk only reads rows at or above its
// own start). With a shared prefix of S blocks the destinations [S*b, k) are
// fresh target blocks and the same loop applies.
#include <hip/hip_runtime.h>

#include "zp_device.h"
#include "zp_host.h"

namespace {

constexpr int kThreads = 256;
constexpr int kB = 16;
constexpr int kUnroll = 8;

struct CompactArgs {
  char* kpool;
  char* vpool;
  const int32_t* keep;
  const int32_t* hole;
  const int32_t* n_pinned;
  const int32_t* src_table;
  const int32_t* dst_table;
  int32_t L, NB, Hkv, max_blocks, n_max, k;
};

template <int RB>  // row bytes = head_dim * element size
__global__ __launch_bounds__(kThreads) void compact_kernel(CompactArgs a) {
  constexpr int kPieces = RB / 16;                 // 16-byte pieces per row
  constexpr int kRowsPerChunk = kThreads * kUnroll / kPieces;
  const int u = blockIdx.x >> 1;
  const int which = blockIdx.x & 1;
  const int hole = a.hole[u];
  if (hole < 0) return;  // unit rejected by the score kernel
  const int h = u % a.Hkv;
  const int l = (u / a.Hkv) % a.L;
  const int r = u / (a.Hkv * a.L);
  const int S = a.n_pinned[r];
  const int start = S > 0 ? S * kB : hole;
  const int k = a.k;
  if (start >= k) return;

  char* pool = which ? a.vpool : a.kpool;
  const int64_t tile_bytes = static_cast<int64_t>(kB) * RB;
  char* base = pool + (static_cast<int64_t>(l) * a.NB * a.Hkv + h) * tile_bytes;
  const int64_t block_stride = static_cast<int64_t>(a.Hkv) * tile_bytes;
  const int32_t* keep = a.keep + static_cast<int64_t>(u) * k;
  const int32_t* src_tab = a.src_table + static_cast<int64_t>(r) * a.max_blocks;
  const int32_t* dst_tab = a.dst_table + static_cast<int64_t>(r) * a.n_max;
  const int tid = threadIdx.x;

  for (int c0 = start; c0 < k; c0 += kRowsPerChunk) {
    zpd::u32x4_t v[kUnroll];
    char* dp[kUnroll];
    int src[kUnroll];
    // rows past k are clamped to row k-1 (always valid) and not stored
#pragma unroll
    for (int e = 0; e < kUnroll; ++e)
      src[e] = keep[min(c0 + (tid + e * kThreads) / kPieces, k - 1)];
#pragma unroll
    for (int e = 0; e < kUnroll; ++e) {
      const int idx = tid + e * kThreads;
      const int t = min(c0 + idx / kPieces, k - 1);
      const int piece = idx % kPieces;
      const char* sp = base + src_tab[src[e] / kB] * block_stride +
                       (src[e] % kB) * RB + piece * 16;
      v[e] = *reinterpret_cast<const zpd::u32x4_t*>(sp);
      dp[e] = base + dst_tab[t / kB] * block_stride + (t % kB) * RB + piece * 16;
    }
    zpd::wait_all_memory();
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kUnroll; ++e)
      if (c0 + (tid + e * kThreads) / kPieces < k) *reinterpret_cast<zpd::u32x4_t*>(dp[e]) = v[e];
  }
}

struct GlobalArgs {
  float* glob;
  const int32_t* keep;
  const float* attn;
  const int32_t* slot;
  const int32_t* n_tokens;
  int32_t L, Hkv, n_cap, num_slots, n_max, k;
};

// Global-score update: g'_t = g_{keep[t]} + attn_{keep[t]} for t < k, zero
// for t in [k, n_cap), in place; the whole row is staged in LDS first.
__global__ __launch_bounds__(kThreads) void global_kernel(GlobalArgs a) {
  extern __shared__ float row[];
  const int u = blockIdx.x;
  const int h = u % a.Hkv;
  const int l = (u / a.Hkv) % a.L;
  const int r = u / (a.Hkv * a.L);
  const int n = a.n_tokens[r];
  const int slot = a.slot[r];
  if (n < a.n_max * kB || n > a.n_cap || slot < 0 || slot >= a.num_slots) return;
  const int32_t* keep = a.keep + static_cast<int64_t>(u) * a.k;
  const float* at = a.attn + static_cast<int64_t>(u) * a.n_cap;
  float* g = a.glob + (static_cast<int64_t>(slot) * a.L * a.Hkv + l * a.Hkv + h) * a.n_cap;
  bool bad = false;
  for (int t = threadIdx.x; t < a.k; t += kThreads) bad |= keep[t] < 0 || keep[t] >= n;
  if (__syncthreads_or(bad)) return;
  for (int t = threadIdx.x; t < a.n_cap; t += kThreads) row[t] = g[t];
  __syncthreads();
  for (int t = threadIdx.x; t < a.n_cap; t += kThreads) {
    float val = 0.f;
    if (t < a.k) {
      const int s = keep[t];
      val = row[s] + at[s];
    }
    g[t] = val;
  }
}

}  // namespace

namespace zp {

zp_status launch_compact(const CompressGeom& g, const zp_kv_pool& pool,
                         const zp_batch& batch, const int32_t* keep,
                         const int32_t* hole, int32_t* err, void* stream) {
  (void)err;
  CompactArgs a;
  a.kpool = static_cast<char*>(pool.k);
  a.vpool = static_cast<char*>(pool.v);
  a.keep = keep;
  a.hole = hole;
  a.n_pinned = batch.n_pinned;
  a.src_table = batch.src_table;
  a.dst_table = batch.dst_table;
  a.L = g.L;
  a.NB = g.num_blocks;
  a.Hkv = g.Hkv;
  a.max_blocks = g.max_blocks;
  a.n_max = g.n_max;
  a.k = g.k;
  const int rb = g.d * (g.dtype == ZP_BF16 ? 2 : 4);
  const unsigned grid = static_cast<unsigned>(g.R) * g.L * g.Hkv * 2u;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (rb) {
    case 128: hipLaunchKernelGGL(compact_kernel<128>, dim3(grid), dim3(kThreads), 0, s, a); break;
    case 256: hipLaunchKernelGGL(compact_kernel<256>, dim3(grid), dim3(kThreads), 0, s, a); break;
    case 512: hipLaunchKernelGGL(compact_kernel<512>, dim3(grid), dim3(kThreads), 0, s, a); break;
    default: return fail(ZP_EUNSUPPORTED, "row bytes %d", rb);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(ZP_EHIP, "compact kernel launch: %s", hipGetErrorString(e));
  return ZP_OK;
}

zp_status launch_global(const CompressGeom& g, float* global_scores,
                        const zp_batch& batch, const int32_t* keep,
                        const float* attn, void* stream) {
  GlobalArgs a;
  a.glob = global_scores;
  a.keep = keep;
  a.attn = attn;
  a.slot = batch.slot;
  a.n_tokens = batch.n_tokens;
  a.L = g.L;
  a.Hkv = g.Hkv;
  a.n_cap = g.n_cap;
  a.num_slots = g.num_slots;
  a.n_max = g.n_max;
  a.k = g.k;
  const size_t dyn = static_cast<size_t>(g.n_cap) * sizeof(float);
  if (dyn > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(global_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(dyn));
    if (e != hipSuccess)
      return fail(ZP_EHIP, "global kernel attribute: %s", hipGetErrorString(e));
  }
  const unsigned grid = static_cast<unsigned>(g.R) * g.L * g.Hkv;
  hipLaunchKernelGGL(global_kernel, dim3(grid), dim3(kThreads), dyn,
                     static_cast<hipStream_t>(stream), a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(ZP_EHIP, "global kernel launch: %s", hipGetErrorString(e));
  return ZP_OK;
}

}  // namespace zp
