// Compression kernel: one workgroup per (request, layer, KV head) unit
// scores, selects and compacts that unit.
//
// Steps, in the order of the method ([zh] §2.1, [de] §2, [es] §2):
//   phase 1  sweep the unit's keys once through the block table: window
//            logits Q K^T on MFMA, per-row softmax normalisers (sums against
//            a per-row reference, exact online fallback on overflow), and the
//            lightning redundancy of every block from the block's 16x16 key
//            Gram matrix (also MFMA, on the same registers: intra-block
//            similarity only, [zh] §2.1, [fr] §2.E);
//   phase 2  sweep the keys again, recompute the logits and sum the
//            normalised probabilities down each column -> attn_t; combine
//            s_t = w_attn attn_t + w_global g_t - w_red red_t (+inf if pinned);
//   select   keep the k = (N_max-1) b best tokens of the unit ([zh] §2.1):
//            an exact radix select on order-preserving 32-bit score keys,
//            ties broken toward the lower position, then the kept positions
//            are written ascending together with the first evicted one;
//   update   (with ZP_UPDATE_GLOBAL) the unit's global-score row follows
//            its tokens: g'_t = g_{keep[t]} + attn_{keep[t]}, 0 past k;
//   compact  move the kept K and V rows, in order, to logical rows [0, k)
//            through the destination table ([zh] §2.1, §2.2).
// Compaction runs in the same workgroup right after its select, so while
// one CU streams its unit's rows other CUs are in their MFMA/exp sweeps: the
// copy traffic overlaps the scoring work instead of following it.
//
// Organisation (gfx950). A workgroup has KG key groups of two waves: wave w
// is (key group kq = w % KG, row half rg = w / KG); at step s the two waves
// of group kq handle key block KG*s + kq, each for its half of the window
// rows, whose MFMA A fragments stay in registers for the whole unit. KG = 4
// (8 waves, one workgroup per CU) takes units with more than 512 KiB of
// keys; KG = 2 (4 waves, half the ring) puts two units on a CU, so one
// unit's latency-bound phases (set-up, select) and its compaction overlap
// the other's sweeps. Larger units stay at one per CU because the column
// sweep's re-reads of a unit's keys are largely served by the last-level
// cache, which holds one such unit per CU but not two. Key blocks reach LDS
// by direct global->LDS loads (16 bytes per lane, 1 KiB fully coalesced per
// instruction) into a ring of NS slots per key group (NS = 7 for bf16 with
// head_dim 128, so up to five blocks per group are in flight without
// costing registers); each wave of the pair issues half of a block's loads.
// The 16-byte chunks of a block row are XOR-swizzled by row in LDS, so the
// ds_read_b128 fragment reads (lane (j, n) takes row n, chunk group j) hit
// distinct banks. Two steps share one fence: an exact s_waitcnt on the
// wave's own loads plus a raw s_barrier (a __syncthreads would drain every
// load in flight). Two waves share a SIMD, so one's MFMA overlaps the
// other's exp/VALU work. Long contexts (token rows that do not fit beside
// the default 8-wave ring in LDS) take a 5-slot ring. The column sweep runs
// backward: it starts on the blocks the first sweep read last and takes the
// ones still in the ring without reloading them. In the column sweep the
// two waves of a SIMD meet the barrier together, so for two unmasked blocks
// the second block's MFMAs are issued one by one between the first block's
// exponentials (fenced with sched_barrier) instead of all before them.
#include <hip/hip_runtime.h>

#include <cstdlib>

#include "zp_device.h"
#include "zp_host.h"

#define ZP_LDS __attribute__((address_space(3)))

namespace {

using zpd::f32x4_t;
using zpd::Frag;

constexpr int kB = 16;  // block size b (one key tile = one block)

struct ScoreArgs {
  void* kpool;
  void* vpool;
  const void* q_window;
  float* glob;
  const int32_t* slot;
  const int32_t* n_tokens;
  const int32_t* src_table;
  const int32_t* dst_table;
  const int32_t* n_pinned;
  const int32_t* seq_pos;  // ring position base (NULL: n)
  int32_t* keep;
  float* attn;
  float* red;
  float* score;
  int32_t* hole_out;
  int32_t* err;
  int32_t R, L, NB, Hkv, Hq, G, w, wG, n_cap, num_slots, max_blocks, n_max, k;
  uint32_t flags;
  float w_attn, w_global, w_red, sl2;  // sl2 = softmax scale * log2(e)
};

// Workgroup shapes. KG key groups of two waves each (one per row half):
// KG = 4 is one 8-wave workgroup per CU with a 112 KiB key ring; KG = 2 is a
// 4-wave workgroup with a 56 KiB ring, so that two of them (two units) share
// a CU and one's latency-bound phases (set-up, select, compaction) overlap
// the other's sweeps.
constexpr int threads_of(int kg) { return 128 * kg; }
// Ring slots per key group: 4 to 8 slots in about 28 KiB per group.
template <typename E, int D>
constexpr int default_slots() {
  constexpr int n = 28 * 1024 / (16 * D * E::kBytes);
  return n > 8 ? 8 : (n < 4 ? 4 : n);
}
// Long contexts: 5 slots (80 KiB for 4 KiB blocks) leave room for 16384
// token rows beside the ring at every supported window size.
constexpr int kLongSlots = 5;
constexpr size_t kLdsPerCu = 160 * 1024;

// s_waitcnt with vmcnt = n (0..28 or 32), expcnt untouched, lgkmcnt = 0.
__device__ __forceinline__ void wait_vm_lgkm0(int n) {
#define ZP_W(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4))
  switch (n) {
    case 0: ZP_W(0); break;    case 1: ZP_W(1); break;    case 2: ZP_W(2); break;
    case 3: ZP_W(3); break;    case 4: ZP_W(4); break;    case 5: ZP_W(5); break;
    case 6: ZP_W(6); break;    case 7: ZP_W(7); break;    case 8: ZP_W(8); break;
    case 9: ZP_W(9); break;    case 10: ZP_W(10); break;  case 11: ZP_W(11); break;
    case 12: ZP_W(12); break;  case 13: ZP_W(13); break;  case 14: ZP_W(14); break;
    case 15: ZP_W(15); break;  case 16: ZP_W(16); break;  case 17: ZP_W(17); break;
    case 18: ZP_W(18); break;  case 19: ZP_W(19); break;  case 20: ZP_W(20); break;
    case 21: ZP_W(21); break;  case 22: ZP_W(22); break;  case 23: ZP_W(23); break;
    case 24: ZP_W(24); break;  case 25: ZP_W(25); break;  case 26: ZP_W(26); break;
    case 27: ZP_W(27); break;  case 28: ZP_W(28); break;  case 32: ZP_W(32); break;
    default: ZP_W(0); break;
  }
#undef ZP_W
}

// Raw workgroup barrier that keeps LDS accesses in program order around it
// without waiting for outstanding global->LDS loads.
__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <typename E, int D, int NS>
struct TileGeom {
  static constexpr int kRowBytes = D * E::kBytes;          // 128, 256 or 512
  static constexpr int kRowChunks = kRowBytes / 16;         // 8, 16 or 32
  static constexpr int kTileBytes = kB * kRowBytes;         // 2, 4 or 8 KiB
  static constexpr int kLoads = kTileBytes / 1024;          // per block
  static constexpr int kLoadsPerWave = kLoads / 2;          // per wave of a pair
  static constexpr int kSwz = kRowChunks < 16 ? kRowChunks - 1 : 15;
  static constexpr int kRing = NS;  // slots per key group
  static_assert(kLoadsPerWave >= 1, "tile too small");
  static_assert(kRing >= 4 && kRing <= 8, "ring length");
  static_assert((kRing - 1) * kLoadsPerWave <= 28, "wait count range");
  // LDS byte offset of chunk (row, c) inside a slot
  __device__ static constexpr int chunk_off(int row, int c) {
    return row * kRowBytes + ((c ^ (row & kSwz)) << 4);
  }
};

template <typename E, int D, int RT, int NS, int KG>
__global__ __launch_bounds__(threads_of(KG)) __attribute__((amdgpu_waves_per_eu(2)))
void compress_kernel(ScoreArgs a) {
  constexpr int kGroups = KG;              // key groups: block kt goes to group kt mod KG
  constexpr int kWaves = 2 * KG;           // two row halves per group
  constexpr int kThreads = threads_of(KG);
  using FragT = Frag<E, D>;
  using TG = TileGeom<E, D, NS>;
  constexpr int kRows = RT * 16;
  constexpr int RTW = (RT + 1) / 2;     // row tiles of the first row half
  constexpr int kRing = TG::kRing;
  __shared__ __attribute__((aligned(16))) char ring[kGroups][kRing][TG::kTileBytes];
  extern __shared__ float s_tok[];  // [n_cap]: red, then order keys
  __shared__ int tab[1024];
  __shared__ float mprime[kRows];
  __shared__ int rowpos[kRows];
  __shared__ float xchg[kGroups][4][16];
  __shared__ int scratch[16];
  __shared__ int sel[2];
  __shared__ float st_m[kGroups][kRows];  // per-group row statistics
  __shared__ float st_z[kGroups][kRows];
  // The ring is idle during the select (the column sweep ended with all
  // loads landed and a barrier): the per-wave histograms live in it then.
  // (Between the sweeps it is not idle: the column sweep starts on the
  // blocks the first sweep left there.)
  static_assert(kWaves * 257 * 4 <= sizeof(ring), "ring too small to alias");
  uint32_t (*hist)[257] = reinterpret_cast<uint32_t (*)[257]>(&ring[0][0][0]);  // one per wave

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int kq = wave % kGroups, rg = wave / kGroups;
  const int jg = lane >> 4, nl = lane & 15;
  const int u = blockIdx.x;
  const int h = u % a.Hkv;
  const int l = (u / a.Hkv) % a.L;
  const int r = u / (a.Hkv * a.L);
  // this wave's row tiles: [rt0, rt0 + nrt)
  const int rt0 = rg * RTW;
  const int nrt = rg ? RT - RTW : RTW;

  // ---- device-side checks of this unit's tables (no writes on failure)
  const int n = a.n_tokens[r];
  const int slot = a.slot[r];
  const int S = a.n_pinned[r];
  const bool protect = (a.flags & ZP_PROTECT_WINDOW) != 0;
  const bool causal = (a.flags & ZP_NONCAUSAL) == 0;
  const int ring_p = ((a.flags & ZP_WINDOW_RING) && a.seq_pos) ? a.seq_pos[r] : n;
  bool bad = n < a.n_max * kB || n > a.n_cap || (n + kB - 1) / kB > a.max_blocks ||
             (n + kB - 1) / kB > 1024 || slot < 0 || slot >= a.num_slots || S < 0 ||
             S * kB + (protect ? a.w : 0) > a.k || ring_p < a.w;
  const int nt = (n + kB - 1) / kB;
  const int32_t* src_tab = a.src_table + static_cast<int64_t>(r) * a.max_blocks;
  const int32_t* dst_tab = a.dst_table + static_cast<int64_t>(r) * a.n_max;
  if (!bad) {
    for (int j = tid; j < nt; j += kThreads) {
      const int b = src_tab[j];
      bad |= b < 0 || b >= a.NB;
      tab[j] = b;
    }
    for (int j = tid; j < a.n_max; j += kThreads)
      bad |= dst_tab[j] < 0 || dst_tab[j] >= a.NB;
    // a slot names one global-score row, rewritten in place by its request
    for (int j = tid; j < a.R; j += kThreads) bad |= j != r && a.slot[j] == slot;
  }
  if (__syncthreads_or(bad)) {
    if (tid == 0) {  // markers of a rejected unit; nothing else is written
      a.keep[static_cast<int64_t>(u) * a.k] = -1;
      if (a.hole_out) a.hole_out[u] = -1;
      *a.err = ZP_EDEVICE;
    }
    return;
  }

  const char* kbase = static_cast<const char*>(a.kpool) +
                      (static_cast<int64_t>(l) * a.NB * a.Hkv + h) * TG::kTileBytes;
  const int64_t block_stride = static_cast<int64_t>(a.Hkv) * TG::kTileBytes;

  // ---- this wave's window rows as MFMA A fragments
  FragT q[RTW];
  {
    const char* qbase = static_cast<const char*>(a.q_window) +
                        static_cast<int64_t>(slot * a.L + l) * a.w * a.Hq * D * E::kBytes;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int row = (rt0 + rt) * 16 + nl;
      if (rt < nrt && row < a.wG) {
        // window row i is the i-th of the last w queries: row i of a
        // linear window, ring row (P - w + i) mod w of a ring
        const int i0 = row / a.G, g = row - i0 * a.G;
        const int i = (a.flags & ZP_WINDOW_RING) ? (ring_p - a.w + i0) % a.w : i0;
        q[rt].load(qbase + (static_cast<int64_t>(i) * a.Hq + h * a.G + g) * D * E::kBytes +
                   jg * (D / 4) * E::kBytes);
      } else {
        q[rt].zero();
      }
    }
  }
  for (int row = tid; row < kRows; row += kThreads)
    rowpos[row] = row < a.wG ? n - a.w + row / a.G : -1;

  const float sl2 = a.sl2;
  const int nsteps = (nt + kGroups - 1) / kGroups;
  // Sweeps run forward or backward over a key group's blocks; the backward
  // column sweep starts with the blocks the row-statistics sweep read last
  // (the newest of them are still in the ring).
  bool backward = false;
  int last_q = 0;  // last step with a block for this key group (set below)
  auto tile_of = [&](int s) { return (backward ? last_q - s : s) * kGroups + kq; };
  auto tile_masked = [&](int kt) {
    return (kt + 1) * kB > n || (causal && kt * kB + kB - 1 > n - a.w);
  };
  auto entry_ok = [&](int rt, int i, int t) {
    const int p = rowpos[(rt0 + rt) * 16 + jg * 4 + i];
    return t < n && (causal ? t <= p : p >= 0);
  };
  // direct global->LDS loads of this wave's half of the block of step s.
  // Lane offsets inside a block are fixed: the destination of load e is the
  // 16-byte slot inst*64 + lane, which holds chunk (row, pos ^ swz(row)).
  int src_off[TG::kLoadsPerWave];
#pragma unroll
  for (int e = 0; e < TG::kLoadsPerWave; ++e) {
    const int sidx = (rg * TG::kLoadsPerWave + e) * 64 + lane;
    const int row = sidx / TG::kRowChunks, pos = sidx % TG::kRowChunks;
    src_off[e] = row * TG::kRowBytes + ((pos ^ (row & TG::kSwz)) << 4);
  }
  int frag_off[FragT::kChunks];
#pragma unroll
  for (int c = 0; c < FragT::kChunks; ++c)
    frag_off[c] = TG::chunk_off(nl, jg * FragT::kChunks + c);
  // last step that has a block for this key group (-1: none)
  const int last = kq < nt ? (nt - 1 - kq) / kGroups : -1;
  last_q = last;
  struct Acc {
    f32x4_t a[RTW];
    f32x4_t g;
  };
  auto issue = [&](int s, int slot_w) {
    const char* src = kbase + tab[tile_of(s)] * block_stride;
    char* dst = ring[kq][slot_w] + rg * TG::kLoadsPerWave * 1024;
#pragma unroll
    for (int e = 0; e < TG::kLoadsPerWave; ++e)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + src_off[e]),
                                       (ZP_LDS void*)(dst + e * 1024), 16, 0, 0);
  };
  auto read_frag = [&](FragT& f, int slot_r) {
    const char* base = ring[kq][slot_r];
#pragma unroll
    for (int c = 0; c < FragT::kChunks; ++c)
      f.v[c] = *reinterpret_cast<const zpd::u32x4_t*>(base + frag_off[c]);
  };
  // One sweep over this key group's blocks, two blocks (steps 2i and 2i+1)
  // per barrier. Loads run ahead through a ring of kRing slots: the prologue
  // issues steps 0..kRing-3 and iteration i refills the slots of steps 2i-2
  // and 2i-1 with steps 2i+kRing-2 and 2i+kRing-1. At iteration i the wave
  // waits until its own loads of steps <= 2i+1 have landed, meets the other
  // waves (all of their halves landed, all of iteration i-1 done), then
  // issues both blocks' MFMAs before their vector work. after(i) runs right
  // after each barrier (and once more after the last iteration).
  auto wait_land = [&](int target, int issued_max) {
    const int ahead = min(issued_max, last) - target;  // later steps in flight
    if (ahead >= kRing - 4) {
      wait_vm_lgkm0((kRing - 4) * TG::kLoadsPerWave);
    } else {
#pragma unroll
      for (int d = kRing - 5; d >= 1; --d)
        if (ahead == d) wait_vm_lgkm0(d * TG::kLoadsPerWave);
      if (ahead <= 0) wait_vm_lgkm0(0);
    }
    step_barrier();
  };
  // The block of forward step p sits in slot p mod kRing. A forward sweep
  // leaves the blocks of its last kRing steps in the ring; the backward
  // sweep that follows starts with exactly those blocks (its step s is
  // forward step last - s), so it reads them in place and loads only from
  // its step kRing on. The waits stay exact: every step it does load comes
  // after every step it does not.
  // Slots are walked with counters: up from 0 forward, down from
  // last mod kRing backward.
  auto needs_load = [&](int s) { return s <= last && !(backward && s < kRing); };
  // pair(slot_a, slot_b, sa, sb) may take over both blocks of an iteration
  // (returning true), e.g. to interleave one block's MFMAs with the other's
  // vector work in one straight-line region.
  auto sweep = [&](auto&& mma, auto&& valu, auto&& after, auto&& pair) {
    static_assert(kRing >= 4, "double steps need four ring slots");
    const int base = backward && last >= 0 ? last % kRing : 0;
    auto adv = [&](int slot) {
      return backward ? (slot == 0 ? kRing - 1 : slot - 1) : (slot + 1 == kRing ? 0 : slot + 1);
    };
    int slot_w = base;
    for (int p = 0; p < kRing - 2; ++p) {
      if (needs_load(p)) issue(p, slot_w);
      slot_w = adv(slot_w);
    }
    int slot_r = base;
    const int niters = (nsteps + 1) / 2;
    for (int i = 0; i < niters; ++i) {
      const int sa = 2 * i, sb = 2 * i + 1;
      wait_land(sb, sa + kRing - 3);
      after(i);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (needs_load(sa + kRing - 2 + e)) issue(sa + kRing - 2 + e, slot_w);
        slot_w = adv(slot_w);
      }
      const int slot_b = adv(slot_r);
      if (!pair(slot_r, slot_b, sa, sb)) {
        Acc acc_a, acc_b;
        if (sa <= last) {
          FragT kc;
          read_frag(kc, slot_r);
          mma(kc, sa, acc_a);
        }
        if (sb <= last) {
          FragT kc;
          read_frag(kc, slot_b);
          mma(kc, sb, acc_b);
        }
        if (sa <= last) valu(acc_a, tile_of(sa), sa);
        if (sb <= last) valu(acc_b, tile_of(sb), sb);
      }
      slot_r = adv(slot_b);
    }
    wait_vm_lgkm0(0);
    step_barrier();
    after(niters);
  };
  auto no_after = [](int) {};
  auto no_pair = [](int, int, int, int) { return false; };
  // logits of this wave's rows against one block (plus, when asked, the
  // block's 16x16 key Gram matrix)
  auto logits = [&](const FragT& kc, Acc& acc, bool gram) {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
      acc.a[rt] = rt < nrt ? zpd::mma_rows<E, D>(q[rt], kc, f32x4_t{0.f, 0.f, 0.f, 0.f})
                           : f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (gram) acc.g = zpd::mma_rows<E, D>(kc, kc, f32x4_t{0.f, 0.f, 0.f, 0.f});
  };
  __syncthreads();

  // ---- phase 1: row statistics and lightning redundancy
  // Each wave takes a per-row reference r (exp2 domain) from the maximum of
  // its first key block and accumulates z = sum exp2(x*sl2 - r) with no
  // running maximum. fp32 absorbs any later growth below 2^127; a row whose
  // sum overflows (or that saw no valid key first) sends the unit through
  // the exact online pass below.
  float mr[RTW][4], z[RTW][4];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[rt][i] = 0.f;
      mr[rt][i] = -INFINITY;
    }
  sweep([&](const FragT& kc, int s, Acc& acc) { logits(kc, acc, (s & 1) == rg); },
        [&](Acc& acc, int kt, int s) {  // masked entries of acc become -inf
    const int t = kt * kB + nl;
    if (s == 0) {  // first block of this wave: the references
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          mr[rt][i] = zpd::max16(entry_ok(rt, i, t) ? acc.a[rt][i] * sl2 : -INFINITY);
        }
    }
    // One accumulation path for every block: in a masked block the entries
    // outside the mask become -inf first (exp2 gives 0). (Two paths made the
    // compiler copy every accumulator back after each unmasked block.) A row
    // whose reference is -inf gets NaN or inf either way and takes the exact
    // pass below.
    if (tile_masked(kt)) {
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!entry_ok(rt, i, t)) acc.a[rt][i] = -INFINITY;
    }
    // all exponentials first (independent), then the sums
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc.a[rt][i] = zpd::fast_exp2(fmaf(acc.a[rt][i], sl2, -mr[rt][i]));
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) z[rt][i] += acc.a[rt][i];
    // lightning redundancy of block kt (the pair alternates by step):
    // column sums of the block's cosine matrix
    if ((s & 1) == rg) {
      // squared norms sit on the Gram diagonal: column nl's is element
      // nl & 3 of lane (nl >> 2, nl); cos = g * rsqrt(max(|a|^2 |b|^2, 1e-16))
      // (row rw = 4 jg + i's norm is in lane (jg, rw) of the same lane
      // group, so all five reads take the diagonal directly, in parallel)
      const f32x4_t& gram = acc.g;
      const int di = nl & 3;
      const float own = di == 0 ? gram[0] : di == 1 ? gram[1] : di == 2 ? gram[2] : gram[3];
      const float dg = __shfl(own, (nl >> 2) * 16 + nl, 64);   // |k_nl|^2
      const int cnt = min(kB, n - kt * kB);
      float cs = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rw = jg * 4 + i;
        const float dr = __shfl(own, jg * 20 + i, 64);           // |k_rw|^2
        if (rw != nl && rw < cnt && nl < cnt)
          cs += gram[i] * __builtin_amdgcn_rsqf(fmaxf(dr * dg, 1e-16f));
      }
      cs = zpd::pairsum16(cs);
      cs = zpd::pairsum32(cs);
      // mean over the block's other keys (1/15 for a full block)
      const float inv = cnt == kB ? 1.f / (kB - 1) : (cnt >= 2 ? 1.f / (cnt - 1) : 0.f);
      if (jg == 0 && nl < cnt) s_tok[t] = cs * inv;
    }
  }, no_after, no_pair);
  // the 16 lanes sharing rows share the reference: their sums just add up
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[rt][i] = zpd::sum16(z[rt][i]);
      if (nl == 0 && rt < nrt) {
        st_m[kq][(rt0 + rt) * 16 + jg * 4 + i] = mr[rt][i];
        st_z[kq][(rt0 + rt) * 16 + jg * 4 + i] = z[rt][i];
      }
    }
  __syncthreads();
  bool redo = false;
  for (int row = tid; row < kRows; row += kThreads) {
    float mm = st_m[0][row], zz = st_z[0][row];
    for (int v = 1; v < kGroups; ++v) zpd::merge_stats(mm, zz, st_m[v][row], st_z[v][row], 1.f);
    if (row < a.wG && !(zz > 0.f && zz < INFINITY && mm > -INFINITY)) redo = true;
    // p = exp2(x*sl2 - mprime) is the normalised probability of a row entry
    mprime[row] = (row < a.wG) ? mm + __log2f(zz) : INFINITY;
  }
  if (__syncthreads_or(redo)) {
    // exact pass: per-lane online maximum and sum (keys read once more)
    float m[RTW][4];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m[rt][i] = -INFINITY;
        z[rt][i] = 0.f;
      }
    sweep([&](const FragT& kc, int, Acc& acc) { logits(kc, acc, false); },
          [&](const Acc& acc, int kt, int) {
      const int t = kt * kB + nl;
      const bool masked = tile_masked(kt);
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
        if (rt >= nrt) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (masked && !entry_ok(rt, i, t)) continue;
          const float x = acc.a[rt][i] * sl2;
          const float dl = x - m[rt][i];
          const float e = zpd::fast_exp2(-fabsf(dl));
          const bool up = dl > 0.f;
          z[rt][i] = up ? fmaf(z[rt][i], e, 1.f) : z[rt][i] + e;
          m[rt][i] = up ? x : m[rt][i];
        }
      }
    }, no_after, no_pair);
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const float m2 = zpd::shfl_xor(m[rt][i], o);
          const float z2 = zpd::shfl_xor(z[rt][i], o);
          zpd::merge_stats(m[rt][i], z[rt][i], m2, z2, 1.f);
        }
        if (nl == 0 && rt < nrt) {
          st_m[kq][(rt0 + rt) * 16 + jg * 4 + i] = m[rt][i];
          st_z[kq][(rt0 + rt) * 16 + jg * 4 + i] = z[rt][i];
        }
      }
    __syncthreads();
    for (int row = tid; row < kRows; row += kThreads) {
      float mm = st_m[0][row], zz = st_z[0][row];
      for (int v = 1; v < kGroups; ++v) zpd::merge_stats(mm, zz, st_m[v][row], st_z[v][row], 1.f);
      mprime[row] = (row < a.wG && zz > 0.f) ? mm + __log2f(zz) : INFINITY;
    }
  }
  __syncthreads();

  // ---- phase 2: column means, score combination
  // Each wave sums its half of the rows; the second half's partial column
  // sums reach the first half through LDS one step later, where the token's
  // attention and score are completed.
  float mp[RTW][4];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      mp[rt][i] = rt < nrt ? mprime[(rt0 + rt) * 16 + jg * 4 + i] : INFINITY;
  const float inv_rows = 1.f / static_cast<float>(a.wG);
  const int64_t urow = static_cast<int64_t>(u) * a.n_cap;
  float* grow = a.glob + (static_cast<int64_t>(slot * a.L + l) * a.Hkv + h) * a.n_cap;
  const int pin_lo = S * kB;
  const int pin_hi = protect ? n - a.w : n;
  float cs_prev[2] = {0.f, 0.f};
  // Inside the sweep only stores are issued (a load whose value is needed
  // would have to wait for every key load issued before it): the attention
  // of a block goes straight to the output row, and scores are formed after
  // the sweep. The second row half hands its partial column sums over through
  // xchg (one buffer per step mod 4); the first half completes them one
  // iteration later, after the barrier that orders the two.
  auto finish = [&](int s, float cs) {  // rg == 0, lanes jg == 0
    const int t = tile_of(s) * kB + nl;
    if (t < n) a.attn[urow + t] = (cs + xchg[kq][s & 3][nl]) * inv_rows;
  };
  // this lane's share of the column sums of an unmasked block
  auto colsum = [&](const Acc& acc) {
    float cs = 0.f;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) cs += zpd::fast_exp2(fmaf(acc.a[rt][i], sl2, -mp[rt][i]));
    return cs;
  };
  // whole-column sum of the wave's rows: to xchg (second half) or kept
  auto emit = [&](float cs, int s) {
    cs = zpd::pairsum16(cs);
    cs = zpd::pairsum32(cs);
    if (rg == 1) {
      if (jg == 0) xchg[kq][s & 3][nl] = cs;
    } else {
      cs_prev[s & 1] = cs;
    }
  };
  backward = true;
  sweep([&](const FragT& kc, int, Acc& acc) { logits(kc, acc, false); },
        [&](const Acc& acc, int kt, int s) {
    const int t = kt * kB + nl;
    float cs = 0.f;
    if (!tile_masked(kt)) {
      cs = colsum(acc);
    } else {
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (entry_ok(rt, i, t)) cs += zpd::fast_exp2(fmaf(acc.a[rt][i], sl2, -mp[rt][i]));
    }
    emit(cs, s);
  }, [&](int i) {  // complete the blocks of iteration i-1
    if (i == 0 || rg != 0 || jg != 0) return;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int s = 2 * (i - 1) + e;
      if (s <= last) finish(s, cs_prev[e]);
    }
  }, [&](int slot_a, int slot_b, int sa, int sb) {
    // two unmasked blocks: block b's MFMAs are interleaved with block a's
    // exponentials (the two waves of a SIMD reach this point together, so
    // without it each pays MFMA a, MFMA b, vector a, vector b in series).
    // bf16 only, up to 8 row tiles (beyond that the registers of both blocks
    // do not fit beside it).
    if constexpr (RT > 8 || E::kBytes != 2) {
      return false;
    } else {
      if (sb > last || tile_masked(tile_of(sa)) || tile_masked(tile_of(sb))) return false;
      FragT ka, kb;
      read_frag(ka, slot_a);
      read_frag(kb, slot_b);
      Acc acc_a, acc_b;
      logits(ka, acc_a, false);
      // each of b's MFMAs (k-chunk c of row tile rt, chunk-major so that
      // consecutive MFMAs feed different row tiles' accumulators) is followed
      // by an equal share of a's entries (fma, exp2, add each), taken in the
      // order colsum() sums them; the fences keep that order
      constexpr int kPer = 4 / FragT::kChunks;  // entries of a per MFMA of b
      float ca = 0.f;
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) acc_b.a[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < FragT::kChunks; ++c)
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
          if (rt < nrt)
            acc_b.a[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(zpd::bf16x8_t, q[rt].v[c]),
                __builtin_bit_cast(zpd::bf16x8_t, kb.v[c]), acc_b.a[rt], 0, 0, 0);
#pragma unroll
          for (int x = 0; x < kPer; ++x) {
            const int e = (c * RTW + rt) * kPer + x;  // entry (e / 4, e % 4) of a
            ca += zpd::fast_exp2(fmaf(acc_a.a[e / 4][e % 4], sl2, -mp[e / 4][e % 4]));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      const float cb = colsum(acc_b);
      emit(ca, sa);
      emit(cb, sb);
      return true;
    }
  });
  __syncthreads();  // the attention row is complete (same workgroup, via L2)
  // In chunks of 8 tokens per thread, every load of a chunk is issued before
  // any of its stores (the optional red/score stores would otherwise keep
  // each iteration's loads behind the previous one's stores).
  constexpr int kComb = 8;
  for (int c0 = 0; c0 < n; c0 += kComb * kThreads) {
    float at[kComb], gt[kComb];
#pragma unroll
    for (int j = 0; j < kComb; ++j) {
      const int t = c0 + j * kThreads + tid;
      at[j] = t < n ? a.attn[urow + t] : 0.f;
      gt[j] = t < n ? grow[t] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kComb; ++j) {
      const int t = c0 + j * kThreads + tid;
      if (t < n) {
        const float rd = s_tok[t];
        float sc = fmaf(a.w_attn, at[j], fmaf(a.w_global, gt[j], -a.w_red * rd));
        if (t < pin_lo || t >= pin_hi) sc = INFINITY;
        if (a.red) a.red[urow + t] = rd;
        if (a.score) a.score[urow + t] = sc;
        s_tok[t] = __uint_as_float(zpd::order_key(sc));
      }
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
    for (int i = tid; i < kWaves * 257; i += kThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    for (int t = tid; t < n; t += kThreads) {
      const uint32_t key = keys[t];
      if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // inclusive scan of 256 bins (summed over the waves), 4 per lane
      uint32_t h0 = 0, h1 = 0, h2 = 0, h3 = 0;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) {
        h0 += hist[w2][lane * 4];
        h1 += hist[w2][lane * 4 + 1];
        h2 += hist[w2][lane * 4 + 2];
        h3 += hist[w2][lane * 4 + 3];
      }
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
  const int ties_before = zpd::block_exclusive_scan<kWaves>(my_ties, scratch, &ties_total);
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
  const int off = zpd::block_exclusive_scan<kWaves>(kept, scratch, &kept_total);
  const int hole = zpd::block_min<kWaves>(first_ev, scratch);
  if (kept_total != a.k) {  // cannot happen for a consistent unit
    if (tid == 0) {
      a.keep[static_cast<int64_t>(u) * a.k] = -1;
      if (a.hole_out) a.hole_out[u] = -1;
      *a.err = ZP_EDEVICE;
    }
    return;
  }
  // kept positions, ascending: to the output row and (the keys are no longer
  // read: both scans above passed barriers) to LDS for the compaction
  int32_t* keep_row = a.keep + static_cast<int64_t>(u) * a.k;
  int* keep_l = reinterpret_cast<int*>(s_tok);
  {
    int o = off;
    for (int t = t0; t < t1; ++t)
      if (!((evict >> (t - t0)) & 1ull)) {
        keep_row[o] = t;
        keep_l[o++] = t;
      }
  }
  if (tid == 0 && a.hole_out) a.hole_out[u] = hole;
  __syncthreads();  // keep_l complete

  // ---- optional global-score update, as zp_update_global does it: the
  // row follows its tokens, g'_t = g_{keep[t]} + attn_{keep[t]} for t < k,
  // 0 after. In place, in ascending chunks: a chunk's values are all read
  // before any of them is written, and a later chunk reads only at or above
  // its own start (keep[t] >= t), never what an earlier chunk wrote.
  if (a.flags & ZP_UPDATE_GLOBAL) {
    constexpr int kPer = 8;  // one chunk covers 4096 (8 waves) or 2048 tokens
    for (int c0 = 0; c0 < a.n_cap; c0 += kPer * kThreads) {
      float gv[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int t = c0 + j * kThreads + tid;
        float v = 0.f;
        if (t < a.k) {
          const int sp = keep_l[t];
          v = grow[sp] + a.attn[urow + sp];
        }
        gv[j] = v;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int t = c0 + j * kThreads + tid;
        if (t < a.n_cap) grow[t] = gv[j];
      }
    }
  }

  // ---- compaction: kept K and V rows, in order, to logical rows [0, k)
  // ([zh] §2.1 re-packing into the first N_max-1 blocks; [zh] §2.2 target
  // blocks after a shared prefix). In place the source of row t is
  // keep[t] >= t and rows below the first hole already hold their token.
  // Rows [start, k) go in ascending chunks; every lane finishes all loads of
  // a chunk before any lane stores it, and a later chunk only reads rows at
  // or above its own start, so no row is overwritten before it is read. With
  // a shared prefix the destinations are fresh target blocks. The copy is
  // streamed with nontemporal loads and stores: its rows are touched once,
  // and keeping them out of the caches leaves those to the key sweeps of the
  // units other CUs are scoring.
  const int start = S > 0 ? S * kB : hole;
  int* dtab = reinterpret_cast<int*>(&ring[0][0][0]);  // the ring is idle
  for (int j = tid; j < a.n_max; j += kThreads) dtab[j] = dst_tab[j];
  __syncthreads();
  if (start >= a.k) return;
  constexpr int kPieces = TG::kRowChunks;               // 16-byte pieces per row
  constexpr int kRowsPerPass = kThreads / kPieces;
  constexpr int kPasses = 8;
  constexpr int kRowsPerChunk = kRowsPerPass * kPasses;
  char* kmut = static_cast<char*>(a.kpool) +
               (static_cast<int64_t>(l) * a.NB * a.Hkv + h) * TG::kTileBytes;
  char* vmut = static_cast<char*>(a.vpool) +
               (static_cast<int64_t>(l) * a.NB * a.Hkv + h) * TG::kTileBytes;
  const int piece16 = (tid % kPieces) * 16, prow = tid / kPieces;
  const int k = a.k;
  struct Buf {
    zpd::u32x4_t vk[kPasses], vv[kPasses];
  };
  // rows past k are clamped to row k-1 (always valid) and not stored.
  // Row offsets: a block id (checked, non-negative) times the block stride
  // (Hkv tiles, below 2^32 bytes) in one 32 x 32 -> 64-bit multiply-add; a
  // chunk's LDS lookups are issued together (all positions, then all block
  // ids), so it waits on LDS twice rather than once per row.
  const uint32_t bstride = static_cast<uint32_t>(block_stride);
  auto row_off = [&](int blk, uint32_t slot) {
    return static_cast<uint64_t>(static_cast<uint32_t>(blk)) * bstride +
           (slot * TG::kRowBytes + static_cast<uint32_t>(piece16));
  };
  auto load_chunk = [&](int c0, Buf& bf) {
    int sp[kPasses], blk[kPasses];
#pragma unroll
    for (int e = 0; e < kPasses; ++e) sp[e] = keep_l[min(c0 + e * kRowsPerPass + prow, k - 1)];
#pragma unroll
    for (int e = 0; e < kPasses; ++e) blk[e] = tab[static_cast<uint32_t>(sp[e]) / kB];
#pragma unroll
    for (int e = 0; e < kPasses; ++e) {
      const uint64_t soff = row_off(blk[e], static_cast<uint32_t>(sp[e]) % kB);
      bf.vk[e] = __builtin_nontemporal_load(reinterpret_cast<const zpd::u32x4_t*>(kmut + soff));
      bf.vv[e] = __builtin_nontemporal_load(reinterpret_cast<const zpd::u32x4_t*>(vmut + soff));
    }
  };
  auto store_chunk = [&](int c0, const Buf& bf) {
    int blk[kPasses];
#pragma unroll
    for (int e = 0; e < kPasses; ++e)
      blk[e] = dtab[static_cast<uint32_t>(min(c0 + e * kRowsPerPass + prow, k - 1)) / kB];
    if (c0 + kRowsPerChunk <= k) {  // every row of the chunk is stored
#pragma unroll
      for (int e = 0; e < kPasses; ++e) {
        const uint32_t t = static_cast<uint32_t>(c0 + e * kRowsPerPass + prow);
        const uint64_t doff = row_off(blk[e], t % kB);
        __builtin_nontemporal_store(bf.vk[e], reinterpret_cast<zpd::u32x4_t*>(kmut + doff));
        __builtin_nontemporal_store(bf.vv[e], reinterpret_cast<zpd::u32x4_t*>(vmut + doff));
      }
    } else {
#pragma unroll
      for (int e = 0; e < kPasses; ++e) {
        const int t = c0 + e * kRowsPerPass + prow;
        if (t < k) {
          const uint64_t doff = row_off(blk[e], static_cast<uint32_t>(t) % kB);
          __builtin_nontemporal_store(bf.vk[e], reinterpret_cast<zpd::u32x4_t*>(kmut + doff));
          __builtin_nontemporal_store(bf.vv[e], reinterpret_cast<zpd::u32x4_t*>(vmut + doff));
        }
      }
    }
  };
  // Triple buffered: the loads of the two chunks after this one are in
  // flight while this chunk's are awaited (they read rows at or above their
  // own chunks' starts, which no store of this chunk touches). Loads return
  // in order, so at most 2*kPasses outstanding memory operations per later
  // chunk in flight means this chunk's loads have landed, whatever the order
  // in which earlier stores complete; the raw barrier then holds every lane
  // until all of the chunk is read.
  auto step = [&](int c0, Buf& cur, Buf& nxt2) {
    const bool more1 = c0 + kRowsPerChunk < k;
    const bool more2 = c0 + 2 * kRowsPerChunk < k;
    if (more2) {
      load_chunk(c0 + 2 * kRowsPerChunk, nxt2);
      wait_vm_lgkm0(4 * kPasses);
    } else if (more1) {
      wait_vm_lgkm0(2 * kPasses);
    } else {
      wait_vm_lgkm0(0);
    }
    step_barrier();
    store_chunk(c0, cur);
    return more1;
  };
  static_assert(4 * kPasses == 32, "wait count");
  Buf b0, b1, b2;
  load_chunk(start, b0);
  if (start + kRowsPerChunk < k) load_chunk(start + kRowsPerChunk, b1);
  for (int c0 = start; c0 < k; c0 += 3 * kRowsPerChunk) {
    if (!step(c0, b0, b2)) break;
    if (!step(c0 + kRowsPerChunk, b1, b0)) break;
    if (!step(c0 + 2 * kRowsPerChunk, b2, b1)) break;
  }
}

template <typename E, int D, int RT, int NS, int KG>
zp_status launch_one(const zp::CompressGeom& g, const ScoreArgs& args,
                     void* stream) {
  const size_t dyn = static_cast<size_t>(g.n_cap) * sizeof(float);
  auto kern = compress_kernel<E, D, RT, NS, KG>;
  hipFuncAttributes fa;
  hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern));
  if (e != hipSuccess)
    return zp::fail(ZP_EHIP, "score kernel attributes: %s", hipGetErrorString(e));
  if (fa.sharedSizeBytes + dyn > kLdsPerCu)
    return zp::fail(ZP_EUNSUPPORTED, "n_cap %d: %zu bytes of token scores do not fit "
                    "beside %zu bytes of key ring in LDS", g.n_cap, dyn,
                    static_cast<size_t>(fa.sharedSizeBytes));
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(dyn));
  if (e != hipSuccess)
    return zp::fail(ZP_EHIP, "score kernel attribute: %s", hipGetErrorString(e));
  const unsigned units = static_cast<unsigned>(g.R) * g.L * g.Hkv;
  hipLaunchKernelGGL(kern, dim3(units), dim3(threads_of(KG)), dyn,
                     static_cast<hipStream_t>(stream), args);
  e = hipGetLastError();
  if (e != hipSuccess)
    return zp::fail(ZP_EHIP, "score kernel launch: %s", hipGetErrorString(e));
  return ZP_OK;
}

template <typename E, int D, int RT, int NS, int KG>
size_t lds_bytes(const zp::CompressGeom& g, zp_status* st) {
  hipFuncAttributes fa;
  const hipError_t e = hipFuncGetAttributes(
      &fa, reinterpret_cast<const void*>(compress_kernel<E, D, RT, NS, KG>));
  if (e != hipSuccess) {
    *st = zp::fail(ZP_EHIP, "score kernel attributes: %s", hipGetErrorString(e));
    return 0;
  }
  *st = ZP_OK;
  return fa.sharedSizeBytes + static_cast<size_t>(g.n_cap) * sizeof(float);
}

// Which workgroup shape a launch takes: 0 = by the rule below, 2 or 4 =
// that many key groups (the environment variable ZIPAGE_KEY_GROUPS, read at
// each launch, so that tests can run both shapes on one input).
int forced_key_groups() {
  const char* v = std::getenv("ZIPAGE_KEY_GROUPS");
  if (!v) return 0;
  const int kg = std::atoi(v);
  return kg == 2 || kg == 4 ? kg : 0;
}

// Two units per CU (KG = 2) when a unit's keys are at most 512 KiB and the
// workgroup fits in half of a CU's LDS; otherwise one 8-wave workgroup per
// CU (KG = 4) with the default ring, or the 5-slot ring when the token rows
// do not fit beside it. The column sweep re-reads a unit's keys, mostly
// from the last-level cache while every CU's units fit in it (256 MB): two
// units of 512 KiB per CU are 256 MB across 256 CUs, larger units would
// spill and are slower with two per CU than with one (measured).
template <typename E, int D, int RT>
zp_status launch_ring(const zp::CompressGeom& g, const ScoreArgs& args,
                      void* stream) {
  constexpr int ns = default_slots<E, D>();
  const int forced = forced_key_groups();
  zp_status st = ZP_OK;
  const bool small_keys = static_cast<size_t>(g.n_cap) * D * E::kBytes <= 512 * 1024;
  if (forced == 2 || (forced == 0 && small_keys)) {
    const size_t lds2 = lds_bytes<E, D, RT, ns, 2>(g, &st);
    if (st != ZP_OK) return st;
    if (lds2 <= kLdsPerCu / 2 || (forced == 2 && lds2 <= kLdsPerCu))
      return launch_one<E, D, RT, ns, 2>(g, args, stream);
  }
  if constexpr (ns > kLongSlots) {
    const size_t lds4 = lds_bytes<E, D, RT, ns, 4>(g, &st);
    if (st != ZP_OK) return st;
    if (lds4 > kLdsPerCu) return launch_one<E, D, RT, kLongSlots, 4>(g, args, stream);
  }
  return launch_one<E, D, RT, ns, 4>(g, args, stream);
}

// Window rows are padded to 16, 32, 64, 128 or 192 and split between the
// two row halves; each half keeps its query fragments in registers.
// (fp32 with head_dim 128 stops at 64 rows: beyond that the fragments spill).
template <typename E, int D>
zp_status dispatch_rows(const zp::CompressGeom& g, const ScoreArgs& args,
                        void* stream) {
  const int rt = (g.wG + 15) / 16;
  constexpr int kMaxRT = (E::kBytes * D > 256) ? 4 : 12;
  if (rt > kMaxRT)
    return zp::fail(ZP_EUNSUPPORTED, "window rows w*G = %d exceed %d for this "
                    "element type and head_dim", g.wG, kMaxRT * 16);
  if (rt <= 1) return launch_ring<E, D, 1>(g, args, stream);
  if (rt <= 2) return launch_ring<E, D, 2>(g, args, stream);
  if (rt <= 4) return launch_ring<E, D, 4>(g, args, stream);
  if constexpr (kMaxRT > 4) {
    if (rt <= 8) return launch_ring<E, D, 8>(g, args, stream);
    return launch_ring<E, D, 12>(g, args, stream);
  }
  return zp::fail(ZP_EUNSUPPORTED, "window rows w*G = %d", g.wG);
}

}  // namespace

namespace zp {

zp_status launch_compress(const CompressGeom& g, const zp_kv_pool& pool,
                          const zp_batch& batch, const void* q_window,
                          float* global_scores,
                          const zp_compress_out& out, int32_t* err, void* stream) {
  ScoreArgs a;
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
  a.err = err;
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
