// All-pairs key redundancy, kept as an ablation of the lightning score
// ([zh] §2.1, [fr] §2.E: the original score compared every pair of the
// N*b cached keys, O(N^2 b^2) for N blocks, and could exhaust memory; the
// lightning score keeps only the pairs inside a block, O(N b^2)).
//
// The unit's n x n key Gram matrix is a dense contraction over head_dim, so
// it runs as a tiled product on MFMA. A workgroup of 4 waves owns a panel of
// row tiles (4 per wave for 16-byte-per-lane-chunk fragments, 2 for fp32
// with head_dim 128); their fragments stay in registers while column tiles
// stream past, four per step, through a 3-slot LDS ring filled by direct
// global->LDS loads (each wave loads one tile; rows are XOR-swizzled so the
// fragment reads hit distinct banks). One step costs each wave up to
// 4 x RT tile products against one LDS read of each column tile.
//
// The cosine matrix is symmetric, so every pair of tiles is formed once: a
// panel takes the column tiles from its own first tile on and skips the
// products below the diagonal. A workgroup runs panel p and then panel
// P - 1 - p (a long and a short row of that triangle), so workgroups carry
// about the same work. An off-diagonal product (row tile i, column
// tile j > i) adds its row sums to tile i's tokens and its column sums to
// tile j's, which belong to another wave or panel: all-token sums therefore
// go to red_all by float atomic adds (zeroed before, divided by n - 1 after,
// by two small kernels), so red_all is exact up to the order of fp32
// additions. Diagonal tiles give their rows both sums and the same-block
// sums, which their owner writes directly.
//
// Cosines: cos(i, j) = g_ij / max(|k_i| |k_j|, 1e-8). Wherever every pair of
// a (row tiles, column tile) step clears the clamp -- the wave's smallest
// row norm times the tile's smallest column norm is at least 1e-8 -- the
// row sum is taken as (1/|k_i|) * sum_j g_ij / |k_j|: one FMA per element,
// with 1/|k_i| applied once at the end. Tiles where the clamp may bind, and
// the diagonal tiles (which also give the same-block sums and exclude
// j == i), take the per-element form. Each token gets two means: over the
// other tokens of its block (equal to the lightning score) and over all
// other tokens.
//
// The workgroups of one unit read the same column tiles, so the workgroup
// ids are dealt to XCDs (round robin on the device) such that consecutive
// workgroups of a unit share one XCD and its L2.
#include <hip/hip_runtime.h>

#include "zp_device.h"
#include "zp_host.h"

#define ZP_LDS __attribute__((address_space(3)))

namespace {

using zpd::f32x4_t;
using zpd::Frag;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kB = 16;
constexpr int kRing = 3;
constexpr int kXcds = 8;

struct FullArgs {
  float* red_block;
  float* red_all;
  const void* kpool;
  const int32_t* n_tokens;
  const int32_t* src_table;
  int32_t units, L, NB, Hkv, max_blocks, n_cap, panels;
  int32_t* err;
};

template <typename E, int D>
struct Geo {
  static constexpr int kRowBytes = D * E::kBytes;          // 128, 256 or 512
  static constexpr int kRowChunks = kRowBytes / 16;
  static constexpr int kTileBytes = kB * kRowBytes;        // 2, 4 or 8 KiB
  static constexpr int kLoads = kTileBytes / 1024;          // per tile and wave
  static constexpr int kSwz = kRowChunks < 16 ? kRowChunks - 1 : 15;
  static constexpr int RT = Frag<E, D>::kChunks <= 4 ? 4 : 2;  // row tiles per wave
  static constexpr int kPanelTiles = kWaves * RT;
  // two workgroups per CU, except fp32 with head_dim 128 (its ring fills LDS)
  static constexpr int kWavesPerSimd = kTileBytes > 4096 ? 1 : 2;
  __device__ static constexpr int chunk_off(int row, int c) {
    return row * kRowBytes + ((c ^ (row & kSwz)) << 4);
  }
};

// s_waitcnt: vmcnt = n (0, 2, 4 or 8), expcnt untouched, lgkmcnt = 0.
__device__ __forceinline__ void wait_vm_lgkm0(int n) {
#define ZP_W(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4))
  switch (n) {
    case 2: ZP_W(2); break;
    case 4: ZP_W(4); break;
    case 8: ZP_W(8); break;
    default: ZP_W(0); break;
  }
#undef ZP_W
}

// LDS accesses stay in program order around a raw barrier that does not wait
// for global->LDS loads in flight.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) only
  raw_barrier();
}

template <typename E, int D>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(Geo<E, D>::kWavesPerSimd)))
void redundancy_full_kernel(FullArgs a) {
  using FragT = Frag<E, D>;
  using GE = Geo<E, D>;
  constexpr int RT = GE::RT;
  __shared__ __attribute__((aligned(16))) char ring[kRing][kWaves][GE::kTileBytes];
  __shared__ float cn2[2][kWaves][kB];   // squared norms of the step's columns
  __shared__ float cmin[2][kWaves];      // smallest valid one per tile
  __shared__ float colw[2][kWaves][4][kB];  // each wave's column sums of a step's tiles
  __shared__ float rnorm2[kWaves][RT][kB];  // squared norms of each wave's rows
  __shared__ int tab[1024];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jg = lane >> 4, nl = lane & 15;
  // the grid is a multiple of 8: block b runs on XCD b % 8, and takes logical
  // id (b % 8) * (grid / 8) + b / 8, so consecutive ids share an XCD
  const int per_xcd = gridDim.x / kXcds;
  const int lid = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  // a workgroup takes panels pp and P - 1 - pp, a long and a short row of
  // the triangle of tile pairs, so every workgroup has about the same work
  const int pairs = (a.panels + 1) / 2;
  if (lid >= a.units * pairs) return;
  const int u = lid / pairs, pp = lid - u * pairs;
  const int h = u % a.Hkv;
  const int l = (u / a.Hkv) % a.L;
  const int r = u / (a.Hkv * a.L);
  const int n = a.n_tokens[r];
  const int nt = (n + kB - 1) / kB;
  if (n < 1 || n > a.n_cap || nt > a.max_blocks || nt > 1024) {
    if (tid == 0 && pp == 0) *a.err = ZP_EDEVICE;
    return;
  }
  if (pp * GE::kPanelTiles >= nt) return;  // both panels lie beyond n
  const bool all_pairs = a.red_all != nullptr;
  const int32_t* src_tab = a.src_table + static_cast<int64_t>(r) * a.max_blocks;
  bool bad = false;
  for (int j = tid; j < nt; j += kThreads) {
    const int b = src_tab[j];
    bad |= b < 0 || b >= a.NB;
    tab[j] = b;
  }
  if (__syncthreads_or(bad)) {
    if (tid == 0) *a.err = ZP_EDEVICE;
    return;
  }
  const char* base = static_cast<const char*>(a.kpool) +
                     (static_cast<int64_t>(l) * a.NB * a.Hkv + h) * GE::kTileBytes;
  const int64_t block_stride = static_cast<int64_t>(a.Hkv) * GE::kTileBytes;
  const int64_t urow = static_cast<int64_t>(u) * a.n_cap;

  // One panel: its row tiles against column tiles from its own first tile on
  // (with red_all; without, the diagonal tiles only). Two panels run one
  // after the other: the second issues its first ring loads after every
  // wave has passed the first's closing barrier (its last ring and
  // column-sum reads precede it) and writes column sums only after its own
  // first step's barrier.
  auto run_panel = [&](const int panel) {
    const int tile0 = panel * GE::kPanelTiles;
    const int ct_end = all_pairs ? nt : min(nt, tile0 + GE::kPanelTiles);

    // ---- this wave's row tiles: fragments and squared row norms
    FragT A[RT];
    float rinv[RT][4];
    float rmin2 = INFINITY;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int grt = tile0 + wave * RT + rt;
      const int row = grt * kB + nl;
      if (grt < nt && row < n)
        A[rt].load(base + tab[grt] * block_stride + nl * GE::kRowBytes +
                   jg * (D / 4) * E::kBytes);
      else
        A[rt].zero();
      float own = A[rt].sumsq();
      own = zpd::pairsum32(zpd::pairsum16(own));
      if (grt < nt && row < n) rmin2 = fminf(rmin2, own);
      if (jg == 0) rnorm2[wave][rt][nl] = own;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float r2 = __shfl(own, 4 * jg + i, 64);
        rinv[rt][i] = r2 > 0.f ? __builtin_amdgcn_rsqf(r2) : 0.f;
      }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) rmin2 = fminf(rmin2, zpd::shfl_xor(rmin2, o));

    // ---- column sweep: step s covers column tiles 4s .. 4s+3
    int src_off[GE::kLoads];
#pragma unroll
    for (int e = 0; e < GE::kLoads; ++e) {
      const int sidx = e * 64 + lane;
      const int row = sidx / GE::kRowChunks, pos = sidx % GE::kRowChunks;
      src_off[e] = row * GE::kRowBytes + ((pos ^ (row & GE::kSwz)) << 4);
    }
    int frag_off[FragT::kChunks];
#pragma unroll
    for (int c = 0; c < FragT::kChunks; ++c)
      frag_off[c] = GE::chunk_off(nl, jg * FragT::kChunks + c);
    auto issue = [&](int s) {  // this wave's column tile of step s
      const int ct = tile0 + 4 * s + wave;
      if (ct >= ct_end) return;
      const char* src = base + tab[ct] * block_stride;
      char* dst = ring[s % kRing][wave];
#pragma unroll
      for (int e = 0; e < GE::kLoads; ++e)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + src_off[e]),
                                         (ZP_LDS void*)(dst + e * 1024), 16, 0, 0);
    };
    auto read_frag = [&](FragT& f, int slot, int c) {
      const char* p = ring[slot][c];
#pragma unroll
      for (int k = 0; k < FragT::kChunks; ++k)
        f.v[k] = *reinterpret_cast<const zpd::u32x4_t*>(p + frag_off[k]);
    };

    float fact[RT][4], exact[RT][4], blk[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) fact[rt][i] = exact[rt][i] = blk[rt][i] = 0.f;

    // column sums of step s, after the barrier that follows it: wave w adds
    // the four waves' sums for column tile w of that step to red_all
    auto flush = [&](int s) {
      const int ct = tile0 + 4 * s + wave;
      const int col = ct * kB + lane;
      if (!all_pairs || ct >= ct_end || lane >= kB || col >= n) return;
      const float v = (colw[s & 1][0][wave][lane] + colw[s & 1][1][wave][lane]) +
                      (colw[s & 1][2][wave][lane] + colw[s & 1][3][wave][lane]);
      unsafeAtomicAdd(&a.red_all[urow + col], v);
    };
    const int nsteps = (ct_end - tile0 + 3) / 4;
    issue(0);
    for (int s = 0; s < nsteps; ++s) {
      // the slot step s+1 fills was last read in step s-2, which every wave
      // finished before the barriers of step s-1
      const bool more = s + 1 < nsteps && tile0 + 4 * (s + 1) + wave < ct_end;
      if (s + 1 < nsteps) issue(s + 1);
      wait_vm_lgkm0(more ? GE::kLoads : 0);
      raw_barrier();  // step s's tiles have landed (every wave waited on its own)
      if (s > 0) flush(s - 1);  // step s-1's column sums are complete
      const int slot = s % kRing;
      {
        const int ct = tile0 + 4 * s + wave;
        if (ct < ct_end) {
          FragT f;
          read_frag(f, slot, wave);
          const bool ok = ct * kB + nl < n;
          float sq = ok ? f.sumsq() : 0.f;
          sq = zpd::pairsum32(zpd::pairsum16(sq));
          const float mn = -zpd::max16(-(ok ? sq : INFINITY));  // row minimum
          if (jg == 0) cn2[s & 1][wave][nl] = sq;
          if (lane == 0) cmin[s & 1][wave] = mn;
        }
      }
      lds_barrier();
      // A step whose four column tiles all lie past this wave's row tiles,
      // inside n, and clear the norm clamp needs none of the guards below:
      // it takes one branch-free body in which the next tile's products are
      // issued before this tile's sums, so the MFMA chains overlap the vector
      // work. It adds exactly what the general path adds, in the same order.
      const int ct0 = tile0 + 4 * s;
      bool fast = false;
      if constexpr (E::kBytes == 2) {
        const float cmin4 = fminf(fminf(cmin[s & 1][0], cmin[s & 1][1]),
                                  fminf(cmin[s & 1][2], cmin[s & 1][3]));
        fast = all_pairs && ct0 + 4 <= ct_end && ct0 > tile0 + wave * RT + RT - 1 &&
               (ct0 + 4) * kB <= n && rmin2 * cmin4 >= 1e-16f;
      }
      if (fast) {
        if constexpr (E::kBytes == 2) {
          float cinv4[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) cinv4[c] = __builtin_amdgcn_rsqf(cn2[s & 1][c][nl]);
          f32x4_t g[2][RT];
          auto products = [&](int c) {
            FragT f;
            read_frag(f, slot, c);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) g[c & 1][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < FragT::kChunks; ++k)
#pragma unroll
              for (int rt = 0; rt < RT; ++rt)
                g[c & 1][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(zpd::bf16x8_t, A[rt].v[k]),
                    __builtin_bit_cast(zpd::bf16x8_t, f.v[k]), g[c & 1][rt], 0, 0, 0);
          };
          products(0);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (c + 1 < 4) products(c + 1);
            float colf = 0.f;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                fact[rt][i] = fmaf(g[c & 1][rt][i], cinv4[c], fact[rt][i]);
                colf = fmaf(g[c & 1][rt][i], rinv[rt][i], colf);
              }
            // the column's sum, the same in all four lane groups (each
            // writes it: no branch in this body)
            const float cs = zpd::pairsum32(zpd::pairsum16(colf * cinv4[c]));
            colw[s & 1][wave][c][nl] = cs;
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int ct = tile0 + 4 * s + c;
          if (ct >= ct_end) break;
          const int col = ct * kB + nl;
          const bool ok = col < n;
          FragT f;
          read_frag(f, slot, c);
          if (!ok) f.zero();
          const float c2 = cn2[s & 1][c][nl];
          const bool safe = rmin2 * cmin[s & 1][c] >= 1e-16f;
          const float cinv = (ok && safe) ? __builtin_amdgcn_rsqf(c2) : 0.f;
          // which of this wave's row tiles pair with column tile ct: those at or
          // below it (at it only, without red_all); the others were or will be
          // formed as (ct, row tile) by the owner of ct
          bool use[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const int grt = tile0 + wave * RT + rt;
            use[rt] = grt < nt && (all_pairs ? grt <= ct : grt == ct);
          }
          f32x4_t g[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) g[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          // past the wave's last row tile every row tile pairs with ct (rows
          // beyond n are zero fragments): the products run unguarded
          const bool every = all_pairs && ct >= tile0 + wave * RT + RT - 1;
          if constexpr (E::kBytes == 2) {
            // chunk-major: the RT accumulation chains interleave
            if (every) {
#pragma unroll
              for (int k = 0; k < FragT::kChunks; ++k)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                  g[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      __builtin_bit_cast(zpd::bf16x8_t, A[rt].v[k]),
                      __builtin_bit_cast(zpd::bf16x8_t, f.v[k]), g[rt], 0, 0, 0);
            } else {
#pragma unroll
              for (int rt = 0; rt < RT; ++rt)
                if (use[rt]) g[rt] = zpd::mma_rows<E, D>(A[rt], f, f32x4_t{0.f, 0.f, 0.f, 0.f});
            }
          } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              if (every || use[rt]) g[rt] = zpd::mma_rows<E, D>(A[rt], f, f32x4_t{0.f, 0.f, 0.f, 0.f});
          }
          float colf = 0.f, colx = 0.f;  // this lane's share of column nl's sums
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            if (!use[rt]) continue;
            const int grt = tile0 + wave * RT + rt;
            if (ct != grt && safe) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                fact[rt][i] = fmaf(g[rt][i], cinv, fact[rt][i]);
                colf = fmaf(g[rt][i], rinv[rt][i], colf);
              }
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int row = grt * kB + 4 * jg + i;
                const float r2 = rnorm2[wave][rt][4 * jg + i];
                const float cv = (ok && row != col)
                                     ? g[rt][i] * __builtin_amdgcn_rsqf(fmaxf(r2 * c2, 1e-16f))
                                     : 0.f;
                exact[rt][i] += cv;
                if (ct == grt) blk[rt][i] += cv;
                else colx += cv;
              }
            }
          }
          if (all_pairs) {
            // the 16 rows of a column sit in the four lane groups
            const float cs = zpd::pairsum32(zpd::pairsum16(fmaf(colf, cinv, colx)));
            if (jg == 0) colw[s & 1][wave][c][nl] = cs;
          }
        }
      }
    }
    lds_barrier();  // the last step's column sums are complete
    if (nsteps > 0) flush(nsteps - 1);

    // ---- row sums over the 16 columns a lane group holds: the same-block
    // mean directly, the all-token sum added to red_all
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int grt = tile0 + wave * RT + rt;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fact[rt][i] = zpd::sum16(fact[rt][i]);
        exact[rt][i] = zpd::sum16(exact[rt][i]);
        blk[rt][i] = zpd::sum16(blk[rt][i]);
        const int row = grt * kB + 4 * jg + i;
        if (nl == 0 && grt < nt && row < n) {
          const int cnt = min(kB, n - grt * kB);
          a.red_block[urow + row] = cnt >= 2 ? blk[rt][i] / (cnt - 1) : 0.f;
          if (all_pairs)
            unsafeAtomicAdd(&a.red_all[urow + row], fmaf(fact[rt][i], rinv[rt][i], exact[rt][i]));
        }
      }
    }
  };
  run_panel(pp);
  const int other = a.panels - 1 - pp;
  if (other != pp && other * GE::kPanelTiles < nt) run_panel(other);
}

// rows [0, n) of a unit's red_all: zeroed before the atomic sums, then
// divided by n - 1 (0 for n < 2); one workgroup per unit
__global__ __launch_bounds__(kThreads) void full_rows_kernel(FullArgs a, int finish) {
  const int u = blockIdx.x;
  const int r = u / (a.Hkv * a.L);
  const int n = min(max(a.n_tokens[r], 0), a.n_cap);
  float* row = a.red_all + static_cast<int64_t>(u) * a.n_cap;
  const float inv = n >= 2 ? 1.f / static_cast<float>(n - 1) : 0.f;
  for (int t = threadIdx.x; t < n; t += kThreads) row[t] = finish ? row[t] * inv : 0.f;
}

template <typename E, int D>
zp_status launch_full(FullArgs a, void* stream) {
  a.panels = ((a.n_cap + kB - 1) / kB + Geo<E, D>::kPanelTiles - 1) / Geo<E, D>::kPanelTiles;
  const int64_t work = static_cast<int64_t>(a.units) * ((a.panels + 1) / 2);
  const int64_t grid = (work + kXcds - 1) / kXcds * kXcds;
  if (grid > (1ll << 31) - 1)
    return zp::fail(ZP_EINVAL, "all-pairs redundancy: %lld workgroups",
                    static_cast<long long>(grid));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.red_all)
    hipLaunchKernelGGL(full_rows_kernel, dim3(a.units), dim3(kThreads), 0, st, a, 0);
  hipLaunchKernelGGL((redundancy_full_kernel<E, D>), dim3(static_cast<unsigned>(grid)),
                     dim3(kThreads), 0, st, a);
  if (a.red_all)
    hipLaunchKernelGGL(full_rows_kernel, dim3(a.units), dim3(kThreads), 0, st, a, 1);
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
  a.panels = 0;
  a.err = err;
  if (g.dtype == ZP_BF16) {
    if (g.d == 128) return launch_full<zpd::BF16, 128>(a, stream);
    if (g.d == 64) return launch_full<zpd::BF16, 64>(a, stream);
  } else {
    if (g.d == 128) return launch_full<zpd::F32, 128>(a, stream);
    if (g.d == 64) return launch_full<zpd::F32, 64>(a, stream);
  }
  return fail(ZP_EUNSUPPORTED, "all-pairs redundancy: head_dim %d", g.d);
}

}  // namespace zp
