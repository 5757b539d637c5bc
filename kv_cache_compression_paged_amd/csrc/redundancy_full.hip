// All-pairs key redundancy, kept as an ablation of the lightning score
// ([zh] §2.1, [fr] §2.E: the original score compared every pair of the
// N*b cached keys, O(N^2 b^2) for N blocks, and could exhaust memory; the
// lightning score keeps only the pairs inside a block, O(N b^2)).
//
// Every 16x16 tile of the n x n key Gram matrix is formed on MFMA (the same
// fragment layout as the compression kernel: lane (j, n) holds chunk j of row
// n, so the contraction is exact) and turned into cosines with the norms of
// its rows and columns. Each token gets two means: over the other tokens of
// its block (equal to the lightning score) and over all other tokens. One
// wave owns one row tile and walks every column tile of its unit through the
// block table; waves are independent (no LDS, no barriers).
#include <hip/hip_runtime.h>

#include "zp_device.h"
#include "zp_host.h"

namespace {

using zpd::f32x4_t;
using zpd::Frag;

constexpr int kThreads = 256;
constexpr int kB = 16;

struct FullArgs {
  float* red_block;
  float* red_all;
  const void* kpool;
  const int32_t* n_tokens;
  const int32_t* src_table;
  int32_t units, L, NB, Hkv, max_blocks, n_cap, tiles_per_unit;
  int32_t* err;
};

// squared norm of row nl of a fragment, summed over the four lanes that hold
// its chunks (lanes nl, nl+16, nl+32, nl+48)
template <typename E, int D>
__device__ __forceinline__ float row_norm2(const Frag<E, D>& f) {
  float s = f.sumsq();
  s += zpd::shfl_xor(s, 16);
  s += zpd::shfl_xor(s, 32);
  return s;
}

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void redundancy_full_kernel(FullArgs a) {
  using FragT = Frag<E, D>;
  constexpr int kRowBytes = D * E::kBytes;
  const int lane = threadIdx.x & 63;
  const int jg = lane >> 4, nl = lane & 15;
  const int wid = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (wid >= a.units * a.tiles_per_unit) return;   // grid padding
  const int u = wid / a.tiles_per_unit;
  const int rt = wid - u * a.tiles_per_unit;          // this wave's row tile
  const int h = u % a.Hkv;
  const int l = (u / a.Hkv) % a.L;
  const int r = u / (a.Hkv * a.L);
  const int n = a.n_tokens[r];
  const int nt = (n + kB - 1) / kB;
  if (n < 1 || n > a.n_cap || nt > a.max_blocks) {
    if (lane == 0 && rt == 0) *a.err = ZP_EDEVICE;
    return;
  }
  if (rt >= nt) return;
  const int32_t* tab = a.src_table + static_cast<int64_t>(r) * a.max_blocks;
  bool bad = false;
  for (int j = lane; j < nt; j += 64) bad |= tab[j] < 0 || tab[j] >= a.NB;
  if (__any(bad)) {
    if (lane == 0) *a.err = ZP_EDEVICE;
    return;
  }
  const char* base = static_cast<const char*>(a.kpool) +
                     (static_cast<int64_t>(l) * a.NB * a.Hkv + h) * kB * kRowBytes;
  const int64_t block_stride = static_cast<int64_t>(a.Hkv) * kB * kRowBytes;
  const int chunk_off = jg * (D / 4) * E::kBytes;

  FragT rowf;
  if (rt * kB + nl < n)
    rowf.load(base + tab[rt] * block_stride + nl * kRowBytes + chunk_off);
  else
    rowf.zero();
  // norms of the rows this lane's outputs hold (rows 4 jg + i of the tile)
  const float rn_own = row_norm2<E, D>(rowf);
  float rn[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) rn[i] = __shfl(rn_own, 4 * jg + i, 64);

  float all_sum[4] = {0.f, 0.f, 0.f, 0.f}, blk_sum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int ct = 0; ct < nt; ++ct) {
    FragT colf;
    const int col = ct * kB + nl;
    if (col < n)
      colf.load(base + tab[ct] * block_stride + nl * kRowBytes + chunk_off);
    else
      colf.zero();
    const float cn = row_norm2<E, D>(colf);     // norm^2 of column nl
    const f32x4_t g = zpd::mma_rows<E, D>(rowf, colf, f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rt * kB + 4 * jg + i;
      const float c = (col < n && row != col)
                          ? g[i] * __builtin_amdgcn_rsqf(fmaxf(rn[i] * cn, 1e-16f))
                          : 0.f;
      all_sum[i] += c;
      if (ct == rt) blk_sum[i] += c;
    }
  }
  // sum over the 16 columns of the tile (lanes of one row group)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      all_sum[i] += zpd::shfl_xor(all_sum[i], o);
      blk_sum[i] += zpd::shfl_xor(blk_sum[i], o);
    }
  if (nl == 0) {
    const int cnt = min(kB, n - rt * kB);
    const int64_t urow = static_cast<int64_t>(u) * a.n_cap;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rt * kB + 4 * jg + i;
      if (row >= n) continue;
      a.red_block[urow + row] = cnt >= 2 ? blk_sum[i] / (cnt - 1) : 0.f;
      if (a.red_all) a.red_all[urow + row] = n >= 2 ? all_sum[i] / (n - 1) : 0.f;
    }
  }
}

template <typename E, int D>
zp_status launch_full(const FullArgs& a, unsigned waves, void* stream) {
  const unsigned grid = (waves + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL((redundancy_full_kernel<E, D>), dim3(grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return zp::fail(ZP_EHIP, "all-pairs redundancy launch: %s", hipGetErrorString(e));
  return ZP_OK;
}

}  // namespace

namespace zp {

zp_status launch_redundancy_full(const CompressGeom& g, const zp_kv_pool& pool,
                                 const zp_batch& batch, float* red_block, float* red_all,
                                 int32_t* err, void* stream) {
  FullArgs a;
  a.red_block = red_block;
  a.red_all = red_all;
  a.kpool = pool.k;
  a.n_tokens = batch.n_tokens;
  a.src_table = batch.src_table;
  a.units = g.R * g.L * g.Hkv;
  a.L = g.L;
  a.NB = g.num_blocks;
  a.Hkv = g.Hkv;
  a.max_blocks = g.max_blocks;
  a.n_cap = g.n_cap;
  a.tiles_per_unit = (g.n_cap + kB - 1) / kB;
  a.err = err;
  const int64_t waves64 = static_cast<int64_t>(a.units) * a.tiles_per_unit;
  if (waves64 > (1ll << 31) - 4)
    return fail(ZP_EINVAL, "all-pairs redundancy: %lld waves", static_cast<long long>(waves64));
  const unsigned waves = static_cast<unsigned>(waves64);
  if (g.dtype == ZP_BF16) {
    if (g.d == 128) return launch_full<zpd::BF16, 128>(a, waves, stream);
    if (g.d == 64) return launch_full<zpd::BF16, 64>(a, waves, stream);
  } else {
    if (g.d == 128) return launch_full<zpd::F32, 128>(a, waves, stream);
    if (g.d == 64) return launch_full<zpd::F32, 64>(a, waves, stream);
  }
  return fail(ZP_EUNSUPPORTED, "all-pairs redundancy: head_dim %d", g.d);
}

}  // namespace zp
