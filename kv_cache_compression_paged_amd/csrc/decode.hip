// Paged decode attention: the consumer of the compressed cache. Decoding
// runs PagedAttention over a request's blocks ([zh] §2.3); after a
// compression those are the N_max-1 re-packed blocks plus the tail block.
//
// One wave per (request, layer, KV head) with its G query heads; a workgroup
// holds four independent waves. Per key block (16 keys): logits Q K^T on MFMA
// (query heads padded to 16 rows, same fragment layout as the score kernel),
// an online softmax per head, and P V on the vector ALUs with each lane
// owning one 16-byte chunk of the head dimension for a quarter (or half) of
// the keys, so V rows are read as coalesced 256-byte segments.
#include <hip/hip_runtime.h>

#include <mutex>

#include "zp_device.h"
#include "zp_host.h"

namespace {

using zpd::f32x4_t;
using zpd::Frag;

constexpr int kThreads = 256;
constexpr int kB = 16;

struct DecodeArgs {
  float* out;
  const void* q;
  void* kpool;
  void* vpool;
  const int32_t* tables;
  const int32_t* seq_lens;
  const void* k_new;  // [R][L][Hkv][D] or null: no append
  const void* v_new;
  float* part_acc;    // split partials [unit][split][G][D] (splits > 1)
  float* part_mz;     // [unit][split][G][2]: running max and sum
  int32_t R, L, Hkv, Hq, G, NB, max_blocks, splits;
  float sl2;
};

template <typename E>
__device__ __forceinline__ void unpack16(const zpd::u32x4_t& c, float* f) {
  if constexpr (E::kBytes == 2) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = zpd::bf16_lo(w[e]);
      f[2 * e + 1] = zpd::bf16_hi(w[e]);
    }
  } else {
    f[0] = __uint_as_float(c.x);
    f[1] = __uint_as_float(c.y);
    f[2] = __uint_as_float(c.z);
    f[3] = __uint_as_float(c.w);
  }
}

// One wave per (unit, split). With an append, the new token's K and V rows
// are first written to their slot (position len of the table) and the token
// is attended from the input registers after the cached ones, so the slot is
// never read back. With splits > 1 the wave covers a contiguous range of the
// unit's blocks and leaves its partial (max, sum, P.V) for decode_combine.
template <typename E, int D, int GP>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  using FragT = Frag<E, D>;
  constexpr int VE = 16 / E::kBytes;          // elements per 16-byte chunk
  constexpr int CPR = D * E::kBytes / 16;      // chunks per row
  constexpr int RPI = 64 / CPR;                // rows per wave instruction
  constexpr int KPL = kB / RPI;                // keys per lane per block
  constexpr int kRowBytes = D * E::kBytes;
  const int lane = threadIdx.x & 63;
  const int jg = lane >> 4, nl = lane & 15;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.R * a.L * a.Hkv * a.splits) return;
  const int unit = wid / a.splits, split = wid - unit * a.splits;
  const int h = unit % a.Hkv;
  const int l = (unit / a.Hkv) % a.L;
  const int r = unit / (a.Hkv * a.L);
  const bool append = a.k_new != nullptr;
  const int len = a.seq_lens[r];                 // cached tokens (before an append)
  const int nt = (len + kB - 1) / kB;            // cached blocks
  const int nt_all = (len + (append ? 1 : 0) + kB - 1) / kB;
  const int32_t* tab = a.tables + static_cast<int64_t>(r) * a.max_blocks;
  // device-side checks: bad length or block id -> this unit writes nothing
  bool bad = len < (append ? 0 : 1) || nt_all > a.max_blocks;
  if (!bad)
    for (int j = lane; j < nt_all; j += 64) bad |= tab[j] < 0 || tab[j] >= a.NB;
  if (__any(bad)) return;

  const int64_t tile_bytes = static_cast<int64_t>(kB) * kRowBytes;
  const int64_t layer_head = (static_cast<int64_t>(l) * a.NB * a.Hkv + h) * tile_bytes;
  char* kbase = static_cast<char*>(a.kpool) + layer_head;
  char* vbase = static_cast<char*>(a.vpool) + layer_head;
  const int64_t block_stride = static_cast<int64_t>(a.Hkv) * tile_bytes;
  const int64_t new_off = static_cast<int64_t>(unit) * kRowBytes;  // [R][L][Hkv][D]
  const bool last_split = split == a.splits - 1;
  if (append && last_split && lane < 2 * CPR) {
    // the new token's K and V rows go to their slot in the table
    const int c = lane % CPR;
    const char* src = static_cast<const char*>(lane < CPR ? a.k_new : a.v_new) + new_off + c * 16;
    char* dst = (lane < CPR ? kbase : vbase) + tab[len / kB] * block_stride +
                (len % kB) * kRowBytes + c * 16;
    *reinterpret_cast<zpd::u32x4_t*>(dst) = *reinterpret_cast<const zpd::u32x4_t*>(src);
  }

  FragT qf;
  if (nl < a.G) {
    const char* qp = static_cast<const char*>(a.q) +
                     ((static_cast<int64_t>(r) * a.L + l) * a.Hq + h * a.G + nl) * D *
                         E::kBytes;
    qf.load(qp + jg * (D / 4) * E::kBytes);
  } else {
    qf.zero();
  }

  // running max / sum of the rows this lane's MFMA outputs hold (4j+i)
  float m[4], z[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    z[i] = 0.f;
  }
  const int vchunk = lane % CPR, vq = lane / CPR;
  float acc[GP][VE];
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[g][e] = 0.f;

  // one block of up to 16 keys: rows [0, nvalid) of kblk / vblk
  auto step = [&](const char* kblk, const char* vblk, int nvalid) {
    FragT kf;
    if (nl < nvalid)
      kf.load(kblk + nl * kRowBytes + jg * (D / 4) * E::kBytes);
    else
      kf.zero();
    zpd::u32x4_t vv[KPL];
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
      const int key = s * RPI + vq;
      vv[s] = key < nvalid
                  ? *reinterpret_cast<const zpd::u32x4_t*>(vblk + key * kRowBytes + vchunk * 16)
                  : zpd::u32x4_t{0u, 0u, 0u, 0u};
    }
    const f32x4_t sc = zpd::mma_rows<E, D>(qf, kf, f32x4_t{0.f, 0.f, 0.f, 0.f});
    const bool valid = nl < nvalid;
    float p[4], alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float tm = zpd::max16(valid ? sc[i] : -INFINITY);
      const float mn = fmaxf(m[i], tm);
      alpha[i] = (m[i] == -INFINITY) ? 0.f : zpd::fast_exp2((m[i] - mn) * a.sl2);
      p[i] = valid ? zpd::fast_exp2((sc[i] - mn) * a.sl2) : 0.f;
      const float rs = zpd::sum16(p[i]);
      z[i] = z[i] * alpha[i] + rs;
      m[i] = mn;
    }
    // P V: lane (vchunk, vq) accumulates keys s*RPI+vq for every head g
    // (head g's statistics sit in lane (g >> 2) * 16, element g & 3)
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      const float al = __int_as_float(
          __builtin_amdgcn_readlane(__float_as_int(alpha[g & 3]), (g >> 2) * 16));
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[g][e] *= al;
    }
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
      float vf[VE];
      unpack16<E>(vv[s], vf);
      const int key = s * RPI + vq;
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const float pg = __shfl(p[g & 3], (g >> 2) * 16 + key, 64);
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[g][e] = fmaf(pg, vf[e], acc[g][e]);
      }
    }
  };

  const int per = (nt + a.splits - 1) / a.splits;
  const int kt0 = split * per, kt1 = min(nt, kt0 + per);
  for (int kt = kt0; kt < kt1; ++kt) {
    const int64_t boff = tab[kt] * block_stride;
    step(kbase + boff, vbase + boff, min(kB, len - kt * kB));
  }
  if (append && last_split)
    step(static_cast<const char*>(a.k_new) + new_off,
         static_cast<const char*>(a.v_new) + new_off, 1);

  // sum the key sub-sets held by lanes with the same chunk
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < VE; ++e)
      for (int o = CPR; o < 64; o <<= 1) acc[g][e] += zpd::shfl_xor(acc[g][e], o);
  if (a.splits == 1) {
    float* orow = a.out + (static_cast<int64_t>(r) * a.L + l) * a.Hq * D;
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      const float zg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z[g & 3]), (g >> 2) * 16));
      if (vq == 0 && g < a.G) {
        float* dst = orow + static_cast<int64_t>(h * a.G + g) * D + vchunk * VE;
        const float inv = 1.f / zg;
#pragma unroll
        for (int e = 0; e < VE; e += 4)
          *reinterpret_cast<float4*>(dst + e) =
              make_float4(acc[g][e] * inv, acc[g][e + 1] * inv, acc[g][e + 2] * inv,
                          acc[g][e + 3] * inv);
      }
    }
  } else {
    const int64_t pbase = static_cast<int64_t>(wid) * a.G;
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      const float zg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z[g & 3]), (g >> 2) * 16));
      const float mg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m[g & 3]), (g >> 2) * 16));
      if (vq == 0 && g < a.G) {
        float* dst = a.part_acc + (pbase + g) * D + vchunk * VE;
#pragma unroll
        for (int e = 0; e < VE; e += 4)
          *reinterpret_cast<float4*>(dst + e) =
              make_float4(acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]);
        if (vchunk == 0) {
          a.part_mz[(pbase + g) * 2] = mg;
          a.part_mz[(pbase + g) * 2 + 1] = zg;
        }
      }
    }
  }
}

// Merge of the split partials of one unit: with M = max_s m_s and weights
// c_s = 2^((m_s - M) * scale * log2 e), out = sum_s c_s acc_s / sum_s c_s z_s.
// A split that saw no key has m = -inf and weight 0.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_combine(DecodeArgs a) {
  const int unit = blockIdx.x;
  const int h = unit % a.Hkv;
  const int l = (unit / a.Hkv) % a.L;
  const int r = unit / (a.Hkv * a.L);
  const bool append = a.k_new != nullptr;
  const int len = a.seq_lens[r];
  const int nt_all = (len + (append ? 1 : 0) + kB - 1) / kB;
  if (len < (append ? 0 : 1) || nt_all > a.max_blocks) return;  // skipped unit
  const int32_t* tab = a.tables + static_cast<int64_t>(r) * a.max_blocks;
  bool bad = false;
  for (int j = threadIdx.x; j < nt_all; j += kThreads) bad |= tab[j] < 0 || tab[j] >= a.NB;
  if (__syncthreads_or(bad)) return;
  float* orow = a.out + ((static_cast<int64_t>(r) * a.L + l) * a.Hq + h * a.G) * D;
  for (int idx = threadIdx.x; idx < a.G * D; idx += kThreads) {
    const int g = idx / D, e = idx - g * D;
    float mx = -INFINITY;
    for (int s = 0; s < a.splits; ++s)
      mx = fmaxf(mx, a.part_mz[((static_cast<int64_t>(unit) * a.splits + s) * a.G + g) * 2]);
    float zs = 0.f, as = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const int64_t pi = (static_cast<int64_t>(unit) * a.splits + s) * a.G + g;
      const float ms = a.part_mz[pi * 2];
      if (ms == -INFINITY) continue;
      const float c = zpd::fast_exp2((ms - mx) * a.sl2);
      zs = fmaf(c, a.part_mz[pi * 2 + 1], zs);
      as = fmaf(c, a.part_acc[pi * D + e], as);
    }
    orow[static_cast<int64_t>(g) * D + e] = as / zs;
  }
}

template <typename E, int D>
zp_status launch_d(const zp::DecodeGeom& g, const DecodeArgs& a, void* stream) {
  const unsigned waves = static_cast<unsigned>(g.R) * g.L * g.Hkv * g.splits;
  const unsigned grid = (waves + 3) / 4;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (g.G <= 4)
    hipLaunchKernelGGL((decode_kernel<E, D, 4>), dim3(grid), dim3(kThreads), 0, s, a);
  else if (g.G <= 8)
    hipLaunchKernelGGL((decode_kernel<E, D, 8>), dim3(grid), dim3(kThreads), 0, s, a);
  else if (g.G <= 16)
    hipLaunchKernelGGL((decode_kernel<E, D, 16>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    return zp::fail(ZP_EUNSUPPORTED, "decode: G = %d > 16", g.G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return zp::fail(ZP_EHIP, "decode kernel launch: %s", hipGetErrorString(e));
  if (g.splits > 1) {
    const unsigned units = static_cast<unsigned>(g.R) * g.L * g.Hkv;
    hipLaunchKernelGGL((decode_combine<D>), dim3(units), dim3(kThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess)
      return zp::fail(ZP_EHIP, "decode combine launch: %s", hipGetErrorString(e));
  }
  return ZP_OK;
}

}  // namespace

namespace zp {

zp_status launch_decode(const DecodeGeom& g, const DecodeIO& io, const zp_kv_pool& pool,
                        void* stream) {
  DecodeArgs a;
  a.out = io.out;
  a.q = io.q;
  a.kpool = pool.k;
  a.vpool = pool.v;
  a.tables = io.tables;
  a.seq_lens = io.seq_lens;
  a.k_new = io.k_new;
  a.v_new = io.v_new;
  a.part_acc = io.part_acc;
  a.part_mz = io.part_mz;
  a.R = g.R;
  a.L = g.L;
  a.Hkv = g.Hkv;
  a.Hq = g.Hq;
  a.G = g.G;
  a.NB = g.num_blocks;
  a.max_blocks = g.max_blocks;
  a.splits = g.splits;
  a.sl2 = g.scale_log2;
  if (g.dtype == ZP_BF16) {
    if (g.d == 128) return launch_d<zpd::BF16, 128>(g, a, stream);
    if (g.d == 64) return launch_d<zpd::BF16, 64>(g, a, stream);
  } else {
    if (g.d == 128) return launch_d<zpd::F32, 128>(g, a, stream);
    if (g.d == 64) return launch_d<zpd::F32, 64>(g, a, stream);
  }
  return fail(ZP_EUNSUPPORTED, "decode: head_dim %d", g.d);
}

}  // namespace zp

// ---------------------------------------------------------------------------
// Split-K decode for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops): the split partials live in
// `scratch`, a file-scope device array of ZP_DECODE_STATIC_BYTES that every
// GPU the library runs on holds until the process ends. In host code the
// array's name is only a stand-in symbol, never a device address: the
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per
// device (with that device current) and kept, and only that address is
// passed to the kernels. Nothing in the scratch has to start at zero: every
// split of every unit the merge kernel reads has written its partials
// earlier on the same stream. Calls that overlap on one GPU share the array
// and race.
static __device__ __align__(256) char scratch[ZP_DECODE_STATIC_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

zp_status scratch_on_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return zp::fail(ZP_EHIP, "zp_paged_decode_split_static: hipGetDevice: %s",
                    hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return zp::fail(ZP_EUNSUPPORTED, "zp_paged_decode_split_static: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return zp::fail(ZP_EHIP, "zp_paged_decode_split_static: scratch address: %s",
                      hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return ZP_OK;
}

}  // namespace

extern "C" zp_status zp_paged_decode_split_static(
    float* out, const void* q, const void* k_new, const void* v_new, const zp_kv_pool* pool,
    const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
    int32_t num_reqs, const zp_params* params, int32_t splits, void* stream) {
  if (!pool || !params || num_reqs < 0 || splits < 1 || params->q_heads <= 0 ||
      pool->layers < 1 || pool->head_dim < 1)
    return zp::fail(ZP_EINVAL, "zp_paged_decode_split_static: bad arguments");
  const size_t need = splits > 1 ? zp::decode_ws_bytes(pool, params, num_reqs, splits) : 0;
  if (need > static_cast<size_t>(ZP_DECODE_STATIC_BYTES))
    return zp::fail(ZP_EWORKSPACE, "zp_paged_decode_split_static: %zu bytes of split "
                    "partials exceed the %zu-byte static scratch (use fewer requests "
                    "or splits, or zp_paged_decode_split with a workspace)", need,
                    static_cast<size_t>(ZP_DECODE_STATIC_BYTES));
  void* ws = nullptr;
  if (splits > 1) {
    const zp_status st = scratch_on_current_device(&ws);
    if (st != ZP_OK) return st;
  }
  return zp::decode_common("zp_paged_decode_split_static", out, q, k_new, v_new, pool,
                           block_tables, max_blocks, seq_lens, num_reqs, params, splits, ws,
                           static_cast<size_t>(ZP_DECODE_STATIC_BYTES), stream);
}
