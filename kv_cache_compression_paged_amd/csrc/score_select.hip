// Score and select kernel: one workgroup (4 waves) per (request, layer, KV
// head) unit.
//
// Steps, in the order of the method ([zh] §2.1, [de] §2, [es] §2):
//   phase 1  sweep the unit's keys once through the block table: window
//            logits Q K^T on MFMA, per-row softmax statistics (max and sum,
//            online), and the lightning redundancy of every block from the
//            block's 16x16 key Gram matrix (also MFMA, on the same registers:
//            intra-block similarity only, [zh] §2.1, [fr] §2.E);
//   phase 2  sweep the keys again, recompute the logits and sum the
//            normalised probabilities down each column -> attn_t; combine
//            s_t = w_attn attn_t + w_global g_t - w_red red_t (+inf if pinned);
//   select   keep the k = (N_max-1) b best tokens of the unit ([zh] §2.1):
//            an exact radix select on order-preserving 32-bit score keys,
//            ties broken toward the lower position, then the kept positions
//            are written ascending together with the first evicted one.
//
// Waves split the key blocks (wave v takes blocks v, v+4, ...); each wave
// keeps the whole query window of the unit in registers as MFMA fragments,
// so every key fragment is loaded once per sweep straight from HBM into the
// B operand and used for all window rows. Phase 2 re-reads the keys: the
// column means need every row's normaliser first.
#include <hip/hip_runtime.h>

#include "zp_device.h"
#include "zp_host.h"

namespace {

using zpd::f32x4_t;
using zpd::Frag;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kB = 16;  // block size b (one key tile = one block)

struct ScoreArgs {
  const void* kpool;
  const void* q_window;
  const float* glob;
  const int32_t* slot;
  const int32_t* n_tokens;
  const int32_t* src_table;
  const int32_t* dst_table;
  const int32_t* n_pinned;
  int32_t* keep;
  float* attn;
  float* red;
  float* score;
  int32_t* hole;
  int32_t* hole_out;
  int32_t* err;
  int32_t L, NB, Hkv, Hq, G, w, wG, n_cap, num_slots, max_blocks, n_max, k;
  uint32_t flags;
  float w_attn, w_global, w_red, sl2;  // sl2 = softmax scale * log2(e)
};

template <typename E, int D, int RT>
__global__ __launch_bounds__(kThreads) void score_select_kernel(ScoreArgs a) {
  using FragT = Frag<E, D>;
  constexpr int kRows = RT * 16;
  extern __shared__ float s_tok[];  // [n_cap]: red, then s, then order keys
  __shared__ float st_m[kWaves][kRows];
  __shared__ float st_z[kWaves][kRows];
  __shared__ float mprime[kRows];
  __shared__ int rowpos[kRows];
  __shared__ int scratch[8];
  __shared__ uint32_t hist[256];
  __shared__ int sel[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int jg = lane >> 4, nl = lane & 15;
  const int u = blockIdx.x;
  const int h = u % a.Hkv;
  const int l = (u / a.Hkv) % a.L;
  const int r = u / (a.Hkv * a.L);

  // ---- device-side checks of this unit's tables (no writes on failure)
  const int n = a.n_tokens[r];
  const int slot = a.slot[r];
  const int S = a.n_pinned[r];
  const bool protect = (a.flags & ZP_PROTECT_WINDOW) != 0;
  const bool causal = (a.flags & ZP_NONCAUSAL) == 0;
  bool bad = n < a.n_max * kB || n > a.n_cap || (n + kB - 1) / kB > a.max_blocks ||
             slot < 0 || slot >= a.num_slots || S < 0 ||
             S * kB + (protect ? a.w : 0) > a.k;
  const int nt = (n + kB - 1) / kB;
  const int32_t* src_tab = a.src_table + static_cast<int64_t>(r) * a.max_blocks;
  const int32_t* dst_tab = a.dst_table + static_cast<int64_t>(r) * a.n_max;
  if (!bad) {
    for (int j = tid; j < nt; j += kThreads)
      bad |= src_tab[j] < 0 || src_tab[j] >= a.NB;
    for (int j = tid; j < a.n_max; j += kThreads)
      bad |= dst_tab[j] < 0 || dst_tab[j] >= a.NB;
  }
  if (__syncthreads_or(bad)) {
    if (tid == 0) {
      a.hole[u] = -1;
      *a.err = ZP_EDEVICE;
    }
    return;
  }

  const int64_t tile_elems = static_cast<int64_t>(kB) * D;
  const char* kbase = static_cast<const char*>(a.kpool) +
                      (static_cast<int64_t>(l) * a.NB * a.Hkv + h) * tile_elems *
                          E::kBytes;
  const int64_t block_stride = static_cast<int64_t>(a.Hkv) * tile_elems * E::kBytes;
  const int lane_off = (nl * D + jg * (D / 4)) * E::kBytes;

  // ---- the window rows of this unit as MFMA A fragments
  FragT q[RT];
  {
    const char* qbase = static_cast<const char*>(a.q_window) +
                        static_cast<int64_t>(slot * a.L + l) * a.w * a.Hq * D *
                            E::kBytes;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = rt * 16 + nl;
      if (row < a.wG) {
        const int i = row / a.G, g = row - i * a.G;
        q[rt].load(qbase + (static_cast<int64_t>(i) * a.Hq + h * a.G + g) * D *
                               E::kBytes +
                   jg * (D / 4) * E::kBytes);
      } else {
        q[rt].zero();
      }
    }
  }
  for (int row = tid; row < kRows; row += kThreads)
    rowpos[row] = row < a.wG ? n - a.w + row / a.G : -1;
  __syncthreads();

  const float sl2 = a.sl2;
  auto tile_masked = [&](int kt) {
    return (kt + 1) * kB > n || (causal && kt * kB + kB - 1 > n - a.w);
  };
  auto load_tile = [&](FragT& f, int kt) {
    if (kt < nt) {
      const int blk = __builtin_amdgcn_readfirstlane(src_tab[kt]);
      if (kt * kB + nl < n)
        f.load(kbase + blk * block_stride + lane_off);
      else
        f.zero();
    }
  };

  // ---- phase 1: row statistics and lightning redundancy
  float m[RT][4], z[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[rt][i] = -INFINITY;
      z[rt][i] = 0.f;
    }
  {
    FragT kc, kn;
    load_tile(kc, wave);
    for (int kt = wave; kt < nt; kt += kWaves) {
      load_tile(kn, kt + kWaves);
      f32x4_t acc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt] = zpd::mma_rows<E, D>(q[rt], kc, f32x4_t{0.f, 0.f, 0.f, 0.f});
      const f32x4_t gram =
          zpd::mma_rows<E, D>(kc, kc, f32x4_t{0.f, 0.f, 0.f, 0.f});
      const int t = kt * kB + nl;
      if (!tile_masked(kt)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = acc[rt][i];
            const float dl = x - m[rt][i];
            const float e = zpd::fast_exp2(-fabsf(dl) * sl2);
            const bool up = dl > 0.f;
            z[rt][i] = up ? fmaf(z[rt][i], e, 1.f) : z[rt][i] + e;
            m[rt][i] = up ? x : m[rt][i];
          }
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int p = rowpos[rt * 16 + jg * 4 + i];
            const bool ok = t < n && (causal ? t <= p : p >= 0);
            if (ok) {
              const float x = acc[rt][i];
              const float dl = x - m[rt][i];
              const float e = zpd::fast_exp2(-fabsf(dl) * sl2);
              const bool up = dl > 0.f;
              z[rt][i] = up ? fmaf(z[rt][i], e, 1.f) : z[rt][i] + e;
              m[rt][i] = up ? x : m[rt][i];
            }
          }
      }
      // lightning redundancy of block kt: column sums of the cosine matrix
      {
        float sq = kc.sumsq();
        sq += zpd::shfl_xor(sq, 16);
        sq += zpd::shfl_xor(sq, 32);
        const float nrm = sqrtf(sq);  // norm of key nl (every j holds it)
        const int cnt = min(kB, n - kt * kB);
        float cs = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rw = jg * 4 + i;
          const float nr = __shfl(nrm, rw, 64);
          if (rw != nl && rw < cnt && nl < cnt)
            cs += gram[i] / fmaxf(nr * nrm, 1e-8f);
        }
        cs += zpd::shfl_xor(cs, 16);
        cs += zpd::shfl_xor(cs, 32);
        if (jg == 0 && nl < cnt) s_tok[t] = cnt >= 2 ? cs / (cnt - 1) : 0.f;
      }
      kc = kn;
    }
  }
  // reduce statistics over the 16 lanes that share rows, then over waves
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float m2 = zpd::shfl_xor(m[rt][i], o);
        const float z2 = zpd::shfl_xor(z[rt][i], o);
        zpd::merge_stats(m[rt][i], z[rt][i], m2, z2, sl2);
      }
      if (nl == 0) {
        st_m[wave][rt * 16 + jg * 4 + i] = m[rt][i];
        st_z[wave][rt * 16 + jg * 4 + i] = z[rt][i];
      }
    }
  __syncthreads();
  for (int row = tid; row < kRows; row += kThreads) {
    float mm = st_m[0][row], zz = st_z[0][row];
    for (int v = 1; v < kWaves; ++v) zpd::merge_stats(mm, zz, st_m[v][row], st_z[v][row], sl2);
    // p = exp2(x*sl2 - mprime) is the normalised probability of a row entry
    mprime[row] = (row < a.wG && zz > 0.f) ? mm * sl2 + __log2f(zz) : INFINITY;
  }
  __syncthreads();

  // ---- phase 2: column means, score combination
  float mp[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) mp[rt][i] = mprime[rt * 16 + jg * 4 + i];
  const float inv_rows = 1.f / static_cast<float>(a.wG);
  const int64_t urow = static_cast<int64_t>(u) * a.n_cap;
  const float* grow = a.glob + (static_cast<int64_t>(slot * a.L + l) * a.Hkv + h) * a.n_cap;
  const int pin_lo = S * kB;
  const int pin_hi = protect ? n - a.w : n;
  {
    FragT kc, kn;
    load_tile(kc, wave);
    for (int kt = wave; kt < nt; kt += kWaves) {
      load_tile(kn, kt + kWaves);
      f32x4_t acc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt] = zpd::mma_rows<E, D>(q[rt], kc, f32x4_t{0.f, 0.f, 0.f, 0.f});
      const int t = kt * kB + nl;
      float cs = 0.f;
      if (!tile_masked(kt)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            cs += zpd::fast_exp2(fmaf(acc[rt][i], sl2, -mp[rt][i]));
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int p = rowpos[rt * 16 + jg * 4 + i];
            const bool ok = t < n && (causal ? t <= p : p >= 0);
            if (ok) cs += zpd::fast_exp2(fmaf(acc[rt][i], sl2, -mp[rt][i]));
          }
      }
      cs += zpd::shfl_xor(cs, 16);
      cs += zpd::shfl_xor(cs, 32);
      if (jg == 0 && t < n) {
        const float at = cs * inv_rows;
        const float rd = s_tok[t];
        float s = fmaf(a.w_attn, at, fmaf(a.w_global, grow[t], -a.w_red * rd));
        if (t < pin_lo || t >= pin_hi) s = INFINITY;
        a.attn[urow + t] = at;
        if (a.red) a.red[urow + t] = rd;
        if (a.score) a.score[urow + t] = s;
        s_tok[t] = __uint_as_float(zpd::order_key(s));
      }
      kc = kn;
    }
  }
  __syncthreads();

  // ---- select: evict the E = n - k smallest (key, then higher position)
  const uint32_t* keys = reinterpret_cast<const uint32_t*>(s_tok);
  const int E_total = n - a.k;
  uint32_t prefix = 0, pmask = 0;
  int want = E_total;  // rank (1-based) of the threshold among the remaining
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int t = tid; t < n; t += kThreads) {
      const uint32_t key = keys[t];
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // inclusive scan of 256 bins, 4 per lane
      const uint32_t h0 = hist[lane * 4], h1 = hist[lane * 4 + 1],
                     h2 = hist[lane * 4 + 2], h3 = hist[lane * 4 + 3];
      const uint32_t loc = h0 + h1 + h2 + h3;
      uint32_t x = loc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      const uint32_t before = x - loc;
      const uint32_t c0 = before + h0, c1 = c0 + h1, c2 = c1 + h2, c3 = c2 + h3;
      const uint32_t wnt = static_cast<uint32_t>(want);
      int bin = -1;
      uint32_t below = 0;
      if (before < wnt && wnt <= c0) { bin = lane * 4; below = before; }
      else if (c0 < wnt && wnt <= c1) { bin = lane * 4 + 1; below = c0; }
      else if (c1 < wnt && wnt <= c2) { bin = lane * 4 + 2; below = c1; }
      else if (c2 < wnt && wnt <= c3) { bin = lane * 4 + 3; below = c2; }
      if (bin >= 0) {
        sel[0] = bin;
        sel[1] = static_cast<int>(below);
      }
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(sel[0]) << shift;
    pmask |= 255u << shift;
    want -= sel[1];
    __syncthreads();
  }
  const uint32_t thr = prefix;  // keys below thr are evicted, and the `want`
                                // highest positions among keys equal to thr

  // each thread owns a contiguous run of positions
  const int per = (n + kThreads - 1) / kThreads;
  const int t0 = min(n, tid * per), t1 = min(n, t0 + per);
  int my_ties = 0;
  for (int t = t0; t < t1; ++t) my_ties += keys[t] == thr;
  int ties_total;
  const int ties_before = zpd::block_exclusive_scan(my_ties, scratch, &ties_total);
  const int ties_after = ties_total - ties_before - my_ties;
  uint64_t evict = 0;
  int seen = 0, kept = 0, first_ev = n;
  for (int t = t0; t < t1; ++t) {
    const uint32_t key = keys[t];
    bool ev = key < thr;
    if (key == thr) {
      const int rank_from_top = ties_after + (my_ties - seen - 1);
      ev = rank_from_top < want;
      ++seen;
    }
    if (ev) {
      evict |= 1ull << (t - t0);
      first_ev = min(first_ev, t);
    } else {
      ++kept;
    }
  }
  int kept_total;
  const int off = zpd::block_exclusive_scan(kept, scratch, &kept_total);
  int32_t* keep_row = a.keep + static_cast<int64_t>(u) * a.k;
  if (kept_total == a.k) {
    int o = off;
    for (int t = t0; t < t1; ++t)
      if (!((evict >> (t - t0)) & 1ull)) keep_row[o++] = t;
  }
  const int hole = zpd::block_min(first_ev, scratch);
  if (tid == 0) {
    if (kept_total != a.k) {  // cannot happen for a consistent unit
      a.hole[u] = -1;
      *a.err = ZP_EDEVICE;
    } else {
      a.hole[u] = hole;
      if (a.hole_out) a.hole_out[u] = hole;
    }
  }
}

template <typename E, int D, int RT>
zp_status launch_one(const zp::CompressGeom& g, const ScoreArgs& args,
                     void* stream) {
  const size_t dyn = static_cast<size_t>(g.n_cap) * sizeof(float);
  auto kern = score_select_kernel<E, D, RT>;
  if (dyn > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(dyn));
    if (e != hipSuccess)
      return zp::fail(ZP_EHIP, "score kernel attribute: %s", hipGetErrorString(e));
  }
  const unsigned units = static_cast<unsigned>(g.R) * g.L * g.Hkv;
  hipLaunchKernelGGL(kern, dim3(units), dim3(kThreads), dyn,
                     static_cast<hipStream_t>(stream), args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return zp::fail(ZP_EHIP, "score kernel launch: %s", hipGetErrorString(e));
  return ZP_OK;
}

// Window rows are padded to 16, 32, 64, 128 or 192; the query fragments of
// all rows stay in registers, so fp32 with head_dim 128 stops at 64 rows
// (beyond that the fragments would spill).
template <typename E, int D>
zp_status dispatch_rows(const zp::CompressGeom& g, const ScoreArgs& args,
                        void* stream) {
  const int rt = (g.wG + 15) / 16;
  constexpr int kMaxRT = (E::kBytes * D > 256) ? 4 : 12;
  if (rt > kMaxRT)
    return zp::fail(ZP_EUNSUPPORTED, "window rows w*G = %d exceed %d for this "
                    "element type and head_dim", g.wG, kMaxRT * 16);
  if (rt <= 1) return launch_one<E, D, 1>(g, args, stream);
  if (rt <= 2) return launch_one<E, D, 2>(g, args, stream);
  if (rt <= 4) return launch_one<E, D, 4>(g, args, stream);
  if constexpr (kMaxRT > 4) {
    if (rt <= 8) return launch_one<E, D, 8>(g, args, stream);
    return launch_one<E, D, 12>(g, args, stream);
  }
  return zp::fail(ZP_EUNSUPPORTED, "window rows w*G = %d", g.wG);
}

}  // namespace

namespace zp {

zp_status launch_score_select(const CompressGeom& g, const zp_kv_pool& pool,
                              const zp_batch& batch, const void* q_window,
                              const float* global_scores,
                              const zp_compress_out& out, int32_t* hole,
                              int32_t* err, void* stream) {
  ScoreArgs a;
  a.kpool = pool.k;
  a.q_window = q_window;
  a.glob = global_scores;
  a.slot = batch.slot;
  a.n_tokens = batch.n_tokens;
  a.src_table = batch.src_table;
  a.dst_table = batch.dst_table;
  a.n_pinned = batch.n_pinned;
  a.keep = out.keep_idx;
  a.attn = out.attn;
  a.red = out.red;
  a.score = out.score;
  a.hole = hole;
  a.hole_out = out.first_hole;
  a.err = err;
  a.L = g.L;
  a.NB = g.num_blocks;
  a.Hkv = g.Hkv;
  a.Hq = g.Hq;
  a.G = g.G;
  a.w = g.w;
  a.wG = g.wG;
  a.n_cap = g.n_cap;
  a.num_slots = g.num_slots;
  a.max_blocks = g.max_blocks;
  a.n_max = g.n_max;
  a.k = g.k;
  a.flags = g.flags;
  a.w_attn = g.w_attn;
  a.w_global = g.w_global;
  a.w_red = g.w_red;
  a.sl2 = g.scale_log2;
  if (g.dtype == ZP_BF16) {
    if (g.d == 128) return dispatch_rows<zpd::BF16, 128>(g, a, stream);
    if (g.d == 64) return dispatch_rows<zpd::BF16, 64>(g, a, stream);
  } else {
    if (g.d == 128) return dispatch_rows<zpd::F32, 128>(g, a, stream);
    if (g.d == 64) return dispatch_rows<zpd::F32, 64>(g, a, stream);
  }
  return fail(ZP_EUNSUPPORTED, "head_dim %d", g.d);
}

}  // namespace zp
