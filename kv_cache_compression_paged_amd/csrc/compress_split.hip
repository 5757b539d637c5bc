// Split-unit compression schedule: each (request, layer, KV head) unit is
// spread over P <= 8 workgroups ("parts"), part p owning the key slice
// [p*SLICE, (p+1)*SLICE) of the unit (SLICE = 512 tokens for up to 128 window
// rows, 256 for up to 192). The method's steps are those of the
// one-workgroup schedule ([zh] §2.1, [de] §2, [es] §2; kernels: [zh] §2.3):
// window attention, lightning redundancy, score combination, top-k selection
// with ties toward the lower position, order-keeping compaction and the
// optional global-score update. What changes is where the data lives:
//
//   - a part loads its slice's keys once, into LDS, and keeps them there
//     until it has written its kept K rows to their destinations;
//   - its window logits are exponentiated against per-row slice maxima and
//     stay in registers (128 VGPRs per lane), so the column sums need no
//     second pass over the keys once the per-row normalisers are known;
//   - it reads its slice's V rows into registers before the eviction set is
//     fixed, so every K and V row of the unit crosses HBM once for reading
//     and once for writing, and the keys are not read a second time.
//
// The parts of a unit exchange two things through the workspace:
//   1. per row of the window, L = m + log2(z) of their slice (m the slice
//      maximum of the scaled logits, z the sum of exp2(x - m)); every part
//      combines the P values into the row's normaliser;
//   2. their eviction candidates: the slice's min(E, slice length) first
//      tokens in eviction order (score key ascending, equal keys from the
//      higher position down), with E = n - k. In that strict order the
//      unit's E first tokens are all among the slices' E first ones, so every
//      part selects the unit's exact eviction set from the candidates alone,
//      and every part knows how many candidates each slice posts.
// Every exchanged word is a 64-bit relaxed device-scope atomic that carries
// a tag (the group's unit iteration + 1), so a reader polls each word until
// its tag matches and no release/acquire fence (an L2 write-back) is needed.
//
// Ordering hazards of the in-place compaction, and why they cannot occur:
// destinations of part p lie at or below its own sources and at most E rows
// into part p-1's slice. A part reads its K rows (into LDS), its V rows and
// its global scores (into registers) before it posts its candidates, and no
// part writes before it has every part's candidates. With target blocks
// (shared prefix) destinations alias no source.
//
// Scheduling: a persistent grid of one workgroup per CU forms groups of P as
// the workgroups start: each takes an atomic ticket t and becomes part
// t mod P of group t / P. Group g runs units g, g + NG, g + 2 NG, ... (NG
// groups), its parts in step with each other. Groups form in the order the
// workgroups start, so at most one group is incomplete at a time and its
// parts wait only for the next workgroups of this grid to start, which the
// hardware does as other work on the device drains. (Two such launches that
// share the device can hold every CU between them with one incomplete group
// each; then both wait until the bounded wait below ends.) Each group has
// its own exchange slot; a word's tag
// is the group's unit iteration + 1, and since both exchanges of a unit are
// full barriers of the group, a slot is never rewritten while a part of the
// group may still read its previous contents. Every wait is bounded: past
// the limit the kernel raises an abort flag that all waits also check,
// records ZP_ESYNC and every workgroup returns.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <type_traits>

#include "zp_device.h"
#include "zp_host.h"

#define ZP_LDS __attribute__((address_space(3)))

namespace {

using zpd::f32x4_t;
using zpd::Frag;
using zpd::u32x4_t;

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kB = 16;
constexpr int kMaxParts = 8;
constexpr int kMaxGroups = 256;
constexpr int kMaxRows = 192;
constexpr int kMaxSlice = 512;
constexpr int kSpinLimit = 1 << 22;  // default polls of one wait (each >= ~0.1 us)
constexpr uint32_t kTagBits = 18;    // candidate words: key 32 | pos 14 | tag 18
constexpr uint32_t kTagMask = (1u << kTagBits) - 1u;

// Workspace layout (bytes from the base). [0, 256) is the error word of
// every compression call; the rest is used by this schedule only.
constexpr size_t kCtlOff = 256;   // u32 ticket, u32 abort flag
constexpr size_t kSlotOff = 512;
constexpr size_t kStatsBytes = static_cast<size_t>(kMaxParts) * kMaxRows * 8;
constexpr size_t kCandBytes = static_cast<size_t>(kMaxParts) * kMaxSlice * 8;
constexpr size_t kSlotBytes = kStatsBytes + kCandBytes;
constexpr size_t kSplitWsBytes = kSlotOff + kMaxGroups * kSlotBytes;

struct SplitArgs {
  void* kpool;
  void* vpool;
  const void* q_window;
  float* glob;
  const int32_t* slot;
  const int32_t* n_tokens;
  const int32_t* src_table;
  const int32_t* dst_table;
  const int32_t* n_pinned;
  const int32_t* seq_pos;
  int32_t* keep;
  float* attn;
  float* red;
  float* score;
  int32_t* hole_out;
  int32_t* err;
  char* ws;
  int32_t R, L, NB, Hkv, Hq, G, w, wG, n_cap, num_slots, max_blocks, n_max, k;
  int32_t P, units, groups;
  int32_t spin_limit;  // polls of one wait before the call gives up
  uint32_t flags;
  float w_attn, w_global, w_red, sl2;
};

__device__ __forceinline__ uint64_t xload(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void xstore(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t xload32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls until ready() holds in every lane of the wave (ready() loads what it
// still lacks). Returns false once `limit` polls found it unready or, with
// honor_abort, another workgroup raised the abort flag; then the flag is
// raised here too.
template <typename F>
__device__ __forceinline__ bool wave_poll(F&& ready, uint32_t* abort_flag, int limit,
                                          bool honor_abort = true) {
  for (int it = 0;; ++it) {
    if (__all(ready())) return true;
    if (it >= limit || (honor_abort && xload32(abort_flag) != 0u)) {
      __hip_atomic_store(abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// s_waitcnt vmcnt(0) lgkmcnt(0): every load of this wave has returned.
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(7 << 4); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations (lgkmcnt(0)), not for its global loads. __syncthreads() also
// drains every global load in flight (vmcnt(0)), which would serialise the
// V-row loads and the next unit's key loads with the selection work.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Block-wide reductions over the 8 waves on lds_barrier (scratch: 16 ints).
__device__ __forceinline__ int wg_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  lds_barrier();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = scratch[w];
    if (w < wave) before += t;
    all += t;
  }
  lds_barrier();
  *total = all;
  return before + x - v;
}
__device__ __forceinline__ int wg_min(int v, int* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  if (lane == 0) scratch[wave] = v;
  lds_barrier();
  int r = scratch[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = min(r, scratch[w]);
  lds_barrier();
  return r;
}
__device__ __forceinline__ bool wg_or(bool v, int* scratch) {
  const int any = __any(v) ? 1 : 0;
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = any;
  lds_barrier();
  int r = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) r |= scratch[w];
  lds_barrier();
  return r != 0;
}

template <int D, int RTW>
__global__ __launch_bounds__(kThreads) void split_kernel(SplitArgs a) {
  using FragT = Frag<zpd::BF16, D>;
  constexpr int SB = 32 / RTW;                 // key blocks per slice
  constexpr int SLICE = SB * kB;               // tokens per slice
  constexpr int kRowBytes = D * 2;
  constexpr int kRowChunks = kRowBytes / 16;   // 16-byte chunks per row
  constexpr int kTile = kB * kRowBytes;        // one (block, head) tile
  constexpr int kLoadsPerTile = kTile / 1024;  // 1 KiB global->LDS loads
  constexpr int kSwz = kRowChunks - 1;
  constexpr int kRowsPerPass = kThreads / kRowChunks;
  constexpr int kPasses = SLICE / kRowsPerPass;
  constexpr int kCandPer = kMaxParts * kMaxSlice / kThreads;  // 8
  static_assert(SLICE <= kMaxSlice && SLICE <= kThreads, "slice");
  static_assert(kRowsPerPass % kB == 0, "a pass covers whole tiles");
  static_assert(RTW * kWaves * 16 >= kMaxRows || RTW == 1, "rows");

  __shared__ __attribute__((aligned(16))) char kt[SB * kTile];
  // per-wave partial column sums; before them, the exchanged row statistics
  __shared__ float colpart[kWaves * SLICE];
  static_assert(kMaxParts * kMaxRows <= kWaves * SLICE, "stats staging");
  __shared__ float red_l[SLICE];
  __shared__ int dest_l[SLICE];
  __shared__ float mprime[RTW * kWaves * 16];
  __shared__ int tab[256];
  __shared__ int dtab[256];
  __shared__ uint32_t hist[256];
  __shared__ int scratch[16];
  __shared__ int sh[8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t* ticket = reinterpret_cast<uint32_t*>(a.ws + kCtlOff);
  uint32_t* abort_flag = ticket + 1;
  const bool causal = (a.flags & ZP_NONCAUSAL) == 0;
  const bool protect = (a.flags & ZP_PROTECT_WINDOW) != 0;
  const bool ringw = (a.flags & ZP_WINDOW_RING) != 0;
  const int64_t block_stride = static_cast<int64_t>(a.Hkv) * kTile;

  // global->LDS load offsets inside a tile: LDS 16-byte slot e*64 + lane of
  // the tile holds chunk (row, pos ^ swz(row)), i.e. chunk c of a row sits at
  // LDS position c ^ (row & kSwz), so fragment reads hit distinct banks
  int src_off[kLoadsPerTile];
#pragma unroll
  for (int e = 0; e < kLoadsPerTile; ++e) {
    const int sidx = e * 64 + lane;
    const int row = sidx / kRowChunks, pos = sidx % kRowChunks;
    src_off[e] = row * kRowBytes + ((pos ^ (row & kSwz)) << 4);
  }
  auto chunk_off = [](int row, int c) { return row * kRowBytes + ((c ^ (row & kSwz)) << 4); };

  // Key loads of slice pp of unit uu into kt, global->LDS, in two steps so
  // that the table reads can go out early: fetch_keys_tab reads the unit's
  // token count and this wave's block ids, issue_keys starts the loads.
  // Entries are checked here too: an invalid one is not loaded, and the unit
  // is rejected when it starts. Indices are clamped into the table.
  // One load per wave: lane i < kPerWave reads the id of block i*8 + wave,
  // lane kPerWave the token count (a lane-varying value stays in one VGPR
  // until issue_keys reads its lanes, so nothing waits for it before then).
  constexpr int kPerWave = (SB + kWaves - 1) / kWaves;
  struct KeyTab {
    int v;
  };
  auto fetch_keys_tab = [&](int uu, int pp, KeyTab& kt_) {
    const int rr = uu / (a.Hkv * a.L);
    const int tcap = min(a.max_blocks, 256);
    const int32_t* st = a.src_table + static_cast<int64_t>(rr) * a.max_blocks;
    const int li = min(lane, kPerWave);
    const int32_t* src = li < kPerWave ? st + min(pp * SB + li * kWaves + wave, tcap - 1)
                                       : a.n_tokens + rr;
    kt_.v = *src;
  };
  auto issue_keys = [&](int uu, int pp, const KeyTab& kt_) {
    const int hh = uu % a.Hkv, ll = (uu / a.Hkv) % a.L;
    const char* kb = static_cast<const char*>(a.kpool) +
                     (static_cast<int64_t>(ll) * a.NB * a.Hkv + hh) * kTile;
    const int nn = __builtin_amdgcn_readlane(kt_.v, kPerWave);
    int ntt = nn <= 0 ? 0 : nn / kB + (nn % kB != 0);
    ntt = min(ntt, min(a.max_blocks, 256));
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int b = i * kWaves + wave;
      const int id = __builtin_amdgcn_readlane(kt_.v, i);
      if (b < SB && pp * SB + b < ntt && id >= 0 && id < a.NB) {
        const char* src = kb + id * block_stride;
#pragma unroll
        for (int e = 0; e < kLoadsPerTile; ++e)
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + src_off[e]),
                                           (ZP_LDS void*)(kt + b * kTile + e * 1024), 16, 0, 0);
      }
    }
  };

  // group formation: ticket t makes this workgroup part t mod P of group t / P
  if (tid == 0)
    sh[0] = static_cast<int>(__hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT));
  lds_barrier();
  const int my_ticket = sh[0];
  const int grp = my_ticket / a.P, p = my_ticket - grp * a.P;
  if (grp >= a.groups) return;  // the grid holds whole groups only
  uint64_t* xstats = reinterpret_cast<uint64_t*>(a.ws + kSlotOff + static_cast<size_t>(grp) * kSlotBytes);
  uint64_t* xcand = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(xstats) + kStatsBytes);
  bool prefetched = false;
  int it = 0;

  for (int u = grp; u < a.units; u += a.groups, ++it) {
    // per-unit opaque copies of the lane indices: addresses derived from them
    // are recomputed in each unit instead of being held (and spilled) across
    // the register-heavy logits phase
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int jg = lane >> 4, nl = lane & 15;
    const int h = u % a.Hkv;
    const int l = (u / a.Hkv) % a.L;
    const int r = u / (a.Hkv * a.L);
    const uint32_t tag = static_cast<uint32_t>(it) + 1u;

    if (!prefetched) {
      KeyTab kt0;
      fetch_keys_tab(u, p, kt0);
      issue_keys(u, p, kt0);
    }

    // ---- the unit's tables, checked as the one-workgroup schedule checks
    // them (every part checks all of them, so all parts agree on `bad`)
    const int n = a.n_tokens[r];
    const int slot = a.slot[r];
    const int S = a.n_pinned[r];
    const int ring_p = (ringw && a.seq_pos) ? a.seq_pos[r] : n;
    bool bad = n < a.n_max * kB || n > a.n_cap || (n + kB - 1) / kB > a.max_blocks ||
               slot < 0 || slot >= a.num_slots || S < 0 ||
               S * kB + (protect ? a.w : 0) > a.k || ring_p < a.w;
    const int nt = bad ? 0 : (n + kB - 1) / kB;
    if (!bad) {
      const int32_t* src_tab = a.src_table + static_cast<int64_t>(r) * a.max_blocks;
      const int32_t* dst_tab = a.dst_table + static_cast<int64_t>(r) * a.n_max;
      for (int j = tid; j < nt; j += kThreads) {
        const int b = src_tab[j];
        bad |= b < 0 || b >= a.NB;
        tab[j] = b;
      }
      for (int j = tid; j < a.n_max; j += kThreads) {
        const int b = dst_tab[j];
        bad |= b < 0 || b >= a.NB;
        dtab[j] = b;
      }
      for (int j = tid; j < a.R; j += kThreads) bad |= j != r && a.slot[j] == slot;
    }
    for (int j = tid; j < SLICE; j += kThreads) dest_l[j] = 0;
    if (wg_or(bad, scratch)) {
      if (tid == 0 && p == 0) {  // markers of a rejected unit; nothing else is written
        a.keep[static_cast<int64_t>(u) * a.k] = -1;
        if (a.hole_out) a.hole_out[u] = -1;
        *a.err = ZP_EDEVICE;
      }
      wait_vm0();  // key loads of this unit land before the LDS is reused
      prefetched = false;
      lds_barrier();
      continue;  // every part of the group skips the unit: no exchange
    }

    const int base = p * SLICE;
    const int slice_n = max(0, min(SLICE, n - base));
    const int nb_here = max(0, min(SB, nt - p * SB));
    const int t = base + tid;
    const bool mine = tid < slice_n;
    const int64_t urow = static_cast<int64_t>(u) * a.n_cap;
    float* grow = a.glob + (static_cast<int64_t>(slot * a.L + l) * a.Hkv + h) * a.n_cap;
    const float gv = mine ? grow[t] : 0.f;

    // ---- this wave's window rows (row tiles wave, wave + 8) as MFMA A
    // fragments, and the position each of the lane's rows sits at
    FragT q[RTW];
    int rp[RTW][4];
    const int RT = (a.wG + 15) / 16;
    {
      const char* qbase = static_cast<const char*>(a.q_window) +
                          static_cast<int64_t>(slot * a.L + l) * a.w * a.Hq * D * 2;
#pragma unroll
      for (int i = 0; i < RTW; ++i) {
        const int rt = wave + kWaves * i;
        const int row = rt * 16 + nl;
        if (rt < RT && row < a.wG) {
          const int i0 = row / a.G, g = row - i0 * a.G;
          const int iw = ringw ? (ring_p - a.w + i0) % a.w : i0;
          q[i].load(qbase + (static_cast<int64_t>(iw) * a.Hq + h * a.G + g) * D * 2 +
                    jg * (D / 4) * 2);
        } else {
          q[i].zero();
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rw = rt * 16 + jg * 4 + j;
          rp[i][j] = rw < a.wG ? n - a.w + rw / a.G : -1;
        }
      }
    }
    wait_vm0();
    lds_barrier();  // keys, tables and dest_l ready

    // ---- logits of the slice (MFMA), lightning redundancy of its blocks
    f32x4_t acc[RTW][SB];
#pragma unroll
    for (int b = 0; b < SB; ++b) {
#pragma unroll
      for (int i = 0; i < RTW; ++i) acc[i][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (b < nb_here) {
        FragT kc;
        const char* tb = kt + b * kTile;
#pragma unroll
        for (int c = 0; c < FragT::kChunks; ++c)
          kc.v[c] = *reinterpret_cast<const u32x4_t*>(tb + chunk_off(nl, jg * FragT::kChunks + c));
#pragma unroll
        for (int i = 0; i < RTW; ++i)
          if (wave + kWaves * i < RT) acc[i][b] = zpd::mma_rows<zpd::BF16, D>(q[i], kc, acc[i][b]);
        if ((b & (kWaves - 1)) == wave) {
          // cosine matrix of the block from its Gram matrix; squared norms on
          // the diagonal (column nl's is element nl & 3 of lane (nl >> 2, nl))
          const f32x4_t gram = zpd::mma_rows<zpd::BF16, D>(kc, kc, f32x4_t{0.f, 0.f, 0.f, 0.f});
          const int kb_g = p * SB + b;
          const int di = nl & 3;
          const float own = di == 0 ? gram[0] : di == 1 ? gram[1] : di == 2 ? gram[2] : gram[3];
          const float dg = __shfl(own, (nl >> 2) * 16 + nl, 64);
          const int cnt = min(kB, n - kb_g * kB);
          float cs = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rw = jg * 4 + i;
            const float dr = __shfl(dg, rw, 64);
            if (rw != nl && rw < cnt && nl < cnt)
              cs += gram[i] * __builtin_amdgcn_rsqf(fmaxf(dr * dg, 1e-16f));
          }
          cs = zpd::pairsum16(cs);
          cs = zpd::pairsum32(cs);
          if (jg == 0 && nl < cnt) red_l[b * kB + nl] = cnt >= 2 ? cs / (cnt - 1) : 0.f;
        }
      }
    }

    // ---- masked logits; per-row slice maximum and exp2 sums. Masked entries
    // (past n, or after a row's position) become -inf by a select (a
    // divergent conditional store into the accumulator was observed to leave
    // some of them in place), in the blocks that hold any; the scale goes
    // into the exponent's fma
    const float sl2 = a.sl2;  // > 0
#pragma unroll
    for (int b = 0; b < SB; ++b) {
      const int kb_g = p * SB + b;
      const bool full = b < nb_here && (kb_g + 1) * kB <= n &&
                        (!causal || kb_g * kB + kB - 1 <= n - a.w);
      if (!full) {  // uniform: only blocks that hold masked entries
        const int tt = kb_g * kB + nl;
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool ok = b < nb_here && tt < n && (causal ? tt <= rp[i][j] : rp[i][j] >= 0);
            acc[i][b][j] = ok ? acc[i][b][j] : -INFINITY;
          }
      }
    }
    float mloc[RTW][4];
    float lsum[RTW][4];
#pragma unroll
    for (int i = 0; i < RTW; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float m = -INFINITY;
#pragma unroll
        for (int b = 0; b < SB; ++b) m = fmaxf(m, acc[i][b][j]);
        m = zpd::max16(m);
        const float msc = m * sl2;                 // the maximum, scaled (exp2 domain)
        const float nms = m == -INFINITY ? 0.f : -msc;
        float z = 0.f;
#pragma unroll
        for (int b = 0; b < SB; ++b) {
          const float e = zpd::fast_exp2(fmaf(acc[i][b][j], sl2, nms));  // exp2(-inf) = 0
          acc[i][b][j] = e;
          z += e;
        }
        z = zpd::sum16(z);
        mloc[i][j] = m == -INFINITY ? -INFINITY : msc;
        lsum[i][j] = m == -INFINITY ? -INFINITY : msc + __log2f(z);
      }
    // exchange 1: post this slice's L for the lane's rows
    if (nl == 0) {
#pragma unroll
      for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rw = (wave + kWaves * i) * 16 + jg * 4 + j;
          if (rw < a.wG)
            xstore(xstats + p * kMaxRows + rw,
                   (static_cast<uint64_t>(tag) << 32) | __float_as_uint(lsum[i][j]));
        }
    }
    // read every part's L of every row (staged in colpart as [part][row])
    {
      const int nst = a.P * a.wG;
      constexpr int kPer = (kMaxParts * kMaxRows + kThreads - 1) / kThreads;
      uint64_t v[kPer];
      bool have[kPer];
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        have[e] = tid + e * kThreads >= nst;
        v[e] = 0;
      }
      const bool ok = wave_poll([&]() {
        // all loads first, then the checks: one round trip per poll
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          if (!have[e]) {
            const int idx = tid + e * kThreads;
            const int qp = idx / a.wG, rw = idx - qp * a.wG;
            v[e] = xload(xstats + qp * kMaxRows + rw);
          }
        }
        bool all = true;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          have[e] = have[e] || static_cast<uint32_t>(v[e] >> 32) == tag;
          all &= have[e];
        }
        return all;
      }, abort_flag, a.spin_limit);
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int idx = tid + e * kThreads;
        if (idx < nst) colpart[idx] = __uint_as_float(static_cast<uint32_t>(v[e]));
      }
      if (wg_or(!ok, scratch)) {
        if (tid == 0) *a.err = ZP_ESYNC;
        return;
      }
    }
    for (int rw = tid; rw < RT * 16; rw += kThreads) {
      float mm = -INFINITY;
      if (rw < a.wG) {
        for (int qp = 0; qp < a.P; ++qp) mm = fmaxf(mm, colpart[qp * a.wG + rw]);
        float zz = 0.f;
        for (int qp = 0; qp < a.P; ++qp) {
          const float lv = colpart[qp * a.wG + rw];
          if (lv != -INFINITY) zz += zpd::fast_exp2(lv - mm);
        }
        mm = mm + __log2f(zz);
      }
      mprime[rw] = mm;  // p = exp2(x - mprime) is the normalised probability
    }
    lds_barrier();

    // ---- column sums of the normalised probabilities: attention
    {
      float f[RTW][4];
#pragma unroll
      for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rw = (wave + kWaves * i) * 16 + jg * 4 + j;
          f[i][j] = (rw < a.wG && mloc[i][j] != -INFINITY)
                        ? zpd::fast_exp2(mloc[i][j] - mprime[rw]) : 0.f;
        }
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        float cs = 0.f;
#pragma unroll
        for (int i = 0; i < RTW; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) cs = fmaf(acc[i][b][j], f[i][j], cs);
        cs = zpd::pairsum16(cs);
        cs = zpd::pairsum32(cs);
        if (jg == 0) colpart[wave * SLICE + b * kB + nl] = cs;
      }
    }
    lds_barrier();
    const float inv_rows = 1.f / static_cast<float>(a.wG);
    float at = 0.f;
    if (tid < SLICE) {
      float cs = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) cs += colpart[w2 * SLICE + tid];
      at = cs * inv_rows;
    }
    const int pin_lo = S * kB;
    const int pin_hi = protect ? n - a.w : n;
    uint32_t key = 0xffffffffu;
    if (mine) {
      a.attn[urow + t] = at;
      const float rd = red_l[tid];
      float sc = fmaf(a.w_attn, at, fmaf(a.w_global, gv, -a.w_red * rd));
      if (t < pin_lo || t >= pin_hi) sc = INFINITY;
      if (a.red) a.red[urow + t] = rd;
      if (a.score) a.score[urow + t] = sc;
      key = zpd::order_key(sc);
    }

    // ---- this slice's V rows into registers (all that may move: with
    // targets, rows past the pinned prefix; in place, every row)
    // (the opaque copy keeps the per-pass offsets from being hoisted out of
    // the unit loop, where they would be held, and spilled, across the sweep)
    int prow = tid / kRowChunks;
    asm volatile("" : "+v"(prow));
    const int piece = tid % kRowChunks;
    const int rowoff = (prow % kB) * kRowBytes + piece * 16;  // same in every pass
    const int64_t hoff = (static_cast<int64_t>(l) * a.NB * a.Hkv + h) * kTile;
    char* kmut = static_cast<char*>(a.kpool) + hoff;
    char* vmut = static_cast<char*>(a.vpool) + hoff;
    const int vlo = S > 0 ? S * kB : 0;
    // the next unit's table entries, read before the V rows so that using
    // them later waits for them alone
    KeyTab next_tab;
    const bool has_next = u + a.groups < a.units;
    if (has_next) fetch_keys_tab(u + a.groups, p, next_tab);
    u32x4_t vv[kPasses];
#pragma unroll
    for (int e = 0; e < kPasses; ++e) {
      const int tr = base + e * kRowsPerPass + prow;
      if (tr < n && tr >= vlo)
        vv[e] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
            vmut + tab[tr / kB] * block_stride + rowoff));
      else
        vv[e] = u32x4_t{0u, 0u, 0u, 0u};
    }
    // ---- this slice's K rows into registers as well: the compaction
    // stores them from there, so the next unit's keys can be loaded into the
    // LDS before this unit's stores (global->LDS loads are issued only after
    // the last LDS access of the unit: the compiler would otherwise wait for
    // them before every LDS access in between)
    u32x4_t kk[kPasses];
    {
      const int lds_k0 = (prow / kB) * kTile + chunk_off(prow % kB, piece);
#pragma unroll
      for (int e = 0; e < kPasses; ++e)
        kk[e] = *reinterpret_cast<const u32x4_t*>(kt + lds_k0 + e * (kRowsPerPass / kB) * kTile);
    }

    // ---- radix select over a set of order keys: the key of rank `want`
    // (1-based, ascending). Each thread offers up to kN keys (valid[i]).
    // Leaves the key in *thr and the rank of the threshold among the keys
    // equal to it (the number of them that fall inside the rank) in *rem.
    auto radix_select = [&](auto kN_c, auto&& keyat, int want, uint32_t* thr, int* rem) {
      constexpr int kN = decltype(kN_c)::value;
      uint32_t prefix = 0, pmask = 0;
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        if (tid < 256) hist[tid] = 0;
        lds_barrier();
#pragma unroll
        for (int i = 0; i < kN; ++i) {
          uint32_t kk;
          if (keyat(i, &kk) && (kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1u);
        }
        lds_barrier();
        if (wave == 0) {
          const uint32_t h0 = hist[lane * 4], h1 = hist[lane * 4 + 1];
          const uint32_t h2 = hist[lane * 4 + 2], h3 = hist[lane * 4 + 3];
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
            sh[2] = bin;
            sh[3] = static_cast<int>(below);
          }
        }
        lds_barrier();
        prefix |= static_cast<uint32_t>(sh[2]) << shift;
        pmask |= 255u << shift;
        want -= sh[3];
        lds_barrier();
      }
      *thr = prefix;
      *rem = want;
    };

    // ---- this slice's eviction candidates: its first min(E, slice_n) tokens
    // in eviction order (key ascending, equal keys from the higher position
    // down), so every part knows how many each slice posts
    const int E_total = n - a.k;
    bool cand = mine;
    if (slice_n > E_total) {
      uint32_t thr_p;
      int rem_p;  // keys equal to thr_p that are taken (the highest positions)
      radix_select(std::integral_constant<int, 1>{},
                   [&](int, uint32_t* kk) { *kk = key; return mine; }, E_total, &thr_p, &rem_p);
      const bool tie = mine && key == thr_p;
      int ties_p;
      const int tb = wg_exclusive_scan(tie ? 1 : 0, scratch, &ties_p);
      cand = mine && (key < thr_p || (tie && ties_p - tb - 1 < rem_p));
    }
    int c_p;
    const int cidx = wg_exclusive_scan(cand ? 1 : 0, scratch, &c_p);
    // in place, this slice's V rows (and, above, its global scores) are read
    // before any part can hold all candidates and start writing; this also
    // waits for the next unit's table reads, issued after the V loads
    wait_vm0();
    lds_barrier();
    if (cand)
      xstore(xcand + p * kMaxSlice + cidx,
             (static_cast<uint64_t>(key) << 32) | (static_cast<uint64_t>(t) << kTagBits) |
                 (tag & kTagMask));
    // every part's candidates: thread tid holds the union entries
    // [kCandPer*tid, kCandPer*tid + kCandPer), in position order
    int coff[kMaxParts + 1];
    coff[0] = 0;
#pragma unroll
    for (int qp = 0; qp < kMaxParts; ++qp)
      coff[qp + 1] = coff[qp] + (qp < a.P ? min(E_total, max(0, min(SLICE, n - qp * SLICE))) : 0);
    const int C = coff[kMaxParts];
    uint64_t cw[kCandPer];
    {
      bool have[kCandPer];
#pragma unroll
      for (int e = 0; e < kCandPer; ++e) {
        have[e] = kCandPer * tid + e >= C;
        cw[e] = 0;
      }
      const uint32_t tmask = tag & kTagMask;
      // After posting, only this group's own words decide (its own bounded
      // wait, not another group's abort): a sibling that holds every
      // candidate may already be writing into this part's slice, so giving
      // up because some other group stopped would leave the unit half
      // compacted. If every part posted, every part sees every word and
      // completes the unit; if one did not, no part holds all of them and
      // none writes.
      const bool ok = wave_poll([&]() {
#pragma unroll
        for (int e = 0; e < kCandPer; ++e) {
          if (!have[e]) {
            const int ui = kCandPer * tid + e;
            int qp = 0, lo = 0;
#pragma unroll
            for (int x = 1; x < kMaxParts; ++x)
              if (ui >= coff[x]) {
                qp = x;
                lo = coff[x];
              }
            cw[e] = xload(xcand + qp * kMaxSlice + (ui - lo));
          }
        }
        bool all = true;
#pragma unroll
        for (int e = 0; e < kCandPer; ++e) {
          have[e] = have[e] || static_cast<uint32_t>(cw[e] & kTagMask) == tmask;
          all &= have[e];
        }
        return all;
      }, abort_flag, a.spin_limit, /*honor_abort=*/false);
      if (wg_or(!ok, scratch)) {
        if (tid == 0) *a.err = ZP_ESYNC;
        return;
      }
    }
    // ---- the unit's eviction set: the E first candidates in eviction order
    // (key ascending, equal keys from the higher position down)
    int ev_before = 0, ev_count = 0, first_ev = 0x7fffffff;
    auto mark = [&](int pos) {
      ++ev_count;
      ev_before += pos < base;
      first_ev = min(first_ev, pos);
      if (pos >= base && pos < base + SLICE) dest_l[pos - base] = -1;
    };
    if (C <= kThreads) {
      // few candidates (E = b: 8 slices x 16): thread i ranks candidate i
      // against all of them, read back from LDS (the column sums are done)
      uint64_t* cl = reinterpret_cast<uint64_t*>(colpart);
      static_assert(kThreads * 8 <= sizeof(colpart), "candidate staging");
#pragma unroll
      for (int e = 0; e < kCandPer; ++e)
        if (kCandPer * tid + e < C) cl[kCandPer * tid + e] = cw[e];
      lds_barrier();
      if (tid < C) {
        const uint64_t me = cl[tid];
        const uint32_t km = static_cast<uint32_t>(me >> 32);
        const uint32_t pm = static_cast<uint32_t>(me >> kTagBits) & 0x3fffu;
        int rank = 0;
        for (int j = 0; j < C; ++j) {
          const uint64_t o = cl[j];
          const uint32_t ko = static_cast<uint32_t>(o >> 32);
          const uint32_t po = static_cast<uint32_t>(o >> kTagBits) & 0x3fffu;
          rank += (ko < km || (ko == km && po > pm)) ? 1 : 0;
        }
        if (rank < E_total) mark(static_cast<int>(pm));
      }
    } else {
      uint32_t thr;
      int want_ties;
      radix_select(std::integral_constant<int, kCandPer>{}, [&](int e, uint32_t* kk) {
        *kk = static_cast<uint32_t>(cw[e] >> 32);
        return kCandPer * tid + e < C;
      }, E_total, &thr, &want_ties);
      int my_ties = 0;
#pragma unroll
      for (int e = 0; e < kCandPer; ++e)
        my_ties += (kCandPer * tid + e < C && static_cast<uint32_t>(cw[e] >> 32) == thr);
      int ties_total;
      const int ties_before = wg_exclusive_scan(my_ties, scratch, &ties_total);
      int seen = 0;
#pragma unroll
      for (int e = 0; e < kCandPer; ++e) {
        if (kCandPer * tid + e >= C) continue;
        const uint32_t kk = static_cast<uint32_t>(cw[e] >> 32);
        const int pos = static_cast<int>((cw[e] >> kTagBits) & 0x3fffu);
        bool ev = kk < thr;
        if (kk == thr) {
          const int above = ties_total - (ties_before + seen) - 1;  // ties at higher positions
          ev = above < want_ties;
          ++seen;
        }
        if (ev) mark(pos);
      }
    }
    // both counts in one scan (each at most 4096)
    int packed_total;
    (void)wg_exclusive_scan((ev_count << 16) | ev_before, scratch, &packed_total);
    const int evb_total = packed_total & 0xffff, evc_total = packed_total >> 16;
    const int hole = wg_min(first_ev, scratch);  // also orders dest_l marks
    const bool kept = mine && dest_l[tid] != -1;
    int kept_slice;
    const int kidx = wg_exclusive_scan(kept ? 1 : 0, scratch, &kept_slice);
    const int dest = base - evb_total + kidx;
    if (evc_total != E_total) {  // cannot happen for a consistent unit
      if (tid == 0 && p == 0) {
        a.keep[static_cast<int64_t>(u) * a.k] = -1;
        if (a.hole_out) a.hole_out[u] = -1;
        *a.err = ZP_EDEVICE;
      }
    } else {
      if (tid < SLICE) dest_l[tid] = kept ? dest : -1;
      if (kept) a.keep[static_cast<int64_t>(u) * a.k + dest] = t;
      if (tid == 0 && p == 0 && a.hole_out) a.hole_out[u] = hole;
    }
    lds_barrier();  // dest_l complete

    // ---- compaction: K and V rows from registers to logical rows dest
    // through the destination table; rows that stay are skipped. The
    // destinations are read out of the LDS first; then the next unit's key
    // loads go out, overlapping these stores.
    const bool consistent = evc_total == E_total;
    int dblk[kPasses], drow[kPasses];
#pragma unroll
    for (int e = 0; e < kPasses; ++e) {
      const int rl = e * kRowsPerPass + prow;
      const int tr = base + rl;
      const int dd = dest_l[rl];
      const bool move = consistent && tr < n && dd >= 0 && (S > 0 ? tr >= S * kB : dd != tr);
      dblk[e] = move ? dtab[dd / kB] : -1;
      drow[e] = dd % kB;
    }
    lds_barrier();  // every LDS access of this unit is done
    prefetched = has_next;
    if (has_next) issue_keys(u + a.groups, p, next_tab);
    if (consistent) {
#pragma unroll
      for (int e = 0; e < kPasses; ++e) {
        if (dblk[e] >= 0) {
          const int64_t doff = dblk[e] * block_stride + drow[e] * kRowBytes + piece * 16;
          __builtin_nontemporal_store(kk[e], reinterpret_cast<u32x4_t*>(kmut + doff));
          __builtin_nontemporal_store(vv[e], reinterpret_cast<u32x4_t*>(vmut + doff));
        }
      }
      // global-score update: g'_dest = g_t + attn_t for kept tokens, 0 on
      // [k, n_cap) (each part zeroes the positions of its own slice range)
      if (a.flags & ZP_UPDATE_GLOBAL) {
        if (kept) grow[dest] = gv + at;
        if (tid < SLICE && t >= a.k && t < a.n_cap) grow[t] = 0.f;
      }
    }
  }
}

__global__ void split_prep_kernel(char* ws) {
  // clears everything after the error word: ticket, abort flag and every
  // exchanged word (tag 0 never matches a unit iteration)
  u32x4_t* p = reinterpret_cast<u32x4_t*>(ws + kCtlOff);
  const size_t nvec = (kSplitWsBytes - kCtlOff) / 16;
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < nvec;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = u32x4_t{0u, 0u, 0u, 0u};
}
static_assert((kSplitWsBytes - kCtlOff) % 16 == 0, "workspace tail");

int cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < 64) cached[dev] = cus;
  return cus;
}

template <int D, int RTW>
zp_status launch_split_t(const SplitArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int cus = cu_count();
  if (cus <= 0) return zp::fail(ZP_EHIP, "split schedule: device attribute query failed");
  hipLaunchKernelGGL(split_prep_kernel, dim3(64), dim3(256), 0, s, a.ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return zp::fail(ZP_EHIP, "split prep launch: %s", hipGetErrorString(e));
  const int grid = a.groups * a.P;
  hipLaunchKernelGGL((split_kernel<D, RTW>), dim3(grid), dim3(kThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return zp::fail(ZP_EHIP, "split kernel launch: %s", hipGetErrorString(e));
  return ZP_OK;
}

int split_parts(const zp::CompressGeom& g) {
  const int slice = g.wG <= 128 ? 512 : 256;
  return (g.n_cap + slice - 1) / slice;
}

// Polls of one exchange wait: kSpinLimit, or ZP_SPLIT_SPIN_LIMIT from the
// environment (read at each call, 0..kSpinLimit) so that a test can make the
// waits give up and see the call report ZP_ESYNC with every workgroup exited.
int spin_limit() {
  const char* e = std::getenv("ZP_SPLIT_SPIN_LIMIT");
  if (!e || !*e) return kSpinLimit;
  char* end = nullptr;
  const long v = std::strtol(e, &end, 10);
  if (*end != '\0' || v < 0 || v > kSpinLimit) return kSpinLimit;
  return static_cast<int>(v);
}

// one workgroup per CU, whole groups of P, at most one group per unit
int split_groups(const zp::CompressGeom& g) {
  const int P = split_parts(g);
  const int64_t units = static_cast<int64_t>(g.R) * g.L * g.Hkv;
  int64_t groups = cu_count() / P;
  if (groups > kMaxGroups) groups = kMaxGroups;
  if (groups > units) groups = units;
  return static_cast<int>(groups);
}

}  // namespace


namespace zp {

size_t split_workspace_bytes() { return kSplitWsBytes; }

bool split_eligible(const CompressGeom& g, size_t workspace_bytes) {
  if (!(g.flags & ZP_SPLIT_UNITS)) return false;
  if (g.dtype != ZP_BF16 || (g.d != 64 && g.d != 128)) return false;
  if (g.wG > kMaxRows) return false;
  const int slice = g.wG <= 128 ? 512 : 256;
  if (g.n_cap > kMaxParts * slice) return false;
  if (workspace_bytes < kSplitWsBytes) return false;
  const int64_t units = static_cast<int64_t>(g.R) * g.L * g.Hkv;
  const int groups = split_groups(g);
  if (groups < 1 || units < 1) return false;
  // a group's unit iterations must fit the candidate words' tag
  return (units + groups - 1) / groups + 1 < (1ll << kTagBits);
}

zp_status launch_compress_split(const CompressGeom& g, const zp_kv_pool& pool,
                                const zp_batch& batch, const void* q_window,
                                float* global_scores, const zp_compress_out& out,
                                void* workspace, void* stream) {
  SplitArgs a;
  a.kpool = pool.k;
  a.vpool = pool.v;
  a.q_window = q_window;
  a.glob = global_scores;
  a.slot = batch.slot;
  a.n_tokens = batch.n_tokens;
  a.src_table = batch.src_table;
  a.dst_table = batch.dst_table;
  a.n_pinned = batch.n_pinned;
  a.seq_pos = batch.seq_pos;
  a.keep = out.keep_idx;
  a.attn = out.attn;
  a.red = out.red;
  a.score = out.score;
  a.hole_out = out.first_hole;
  a.err = static_cast<int32_t*>(workspace);
  a.ws = static_cast<char*>(workspace);
  a.R = g.R;
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
  a.P = split_parts(g);
  a.units = g.R * g.L * g.Hkv;
  a.groups = split_groups(g);
  a.spin_limit = spin_limit();
  if (g.wG <= 128) {
    if (g.d == 128) return launch_split_t<128, 1>(a, stream);
    return launch_split_t<64, 1>(a, stream);
  }
  if (g.d == 128) return launch_split_t<128, 2>(a, stream);
  return launch_split_t<64, 2>(a, stream);
}

}  // namespace zp
