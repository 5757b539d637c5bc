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
  const void* kpool;
  const void* vpool;
  const int32_t* tables;
  const int32_t* seq_lens;
  int32_t R, L, Hkv, Hq, G, NB, max_blocks;
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

template <typename E, int D, int GP>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  using FragT = Frag<E, D>;
  constexpr int VE = 16 / E::kBytes;          // elements per 16-byte chunk
  constexpr int CPR = D * E::kBytes / 16;      // chunks per row
  constexpr int RPI = 64 / CPR;                // rows per wave instruction
  constexpr int KPL = kB / RPI;                // keys per lane per block
  const int lane = threadIdx.x & 63;
  const int jg = lane >> 4, nl = lane & 15;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= a.R * a.L * a.Hkv) return;
  const int h = unit % a.Hkv;
  const int l = (unit / a.Hkv) % a.L;
  const int r = unit / (a.Hkv * a.L);
  const int len = a.seq_lens[r];
  const int nt = (len + kB - 1) / kB;
  const int32_t* tab = a.tables + static_cast<int64_t>(r) * a.max_blocks;
  float* orow = a.out + (static_cast<int64_t>(r) * a.L + l) * a.Hq * D;
  // device-side checks: bad length or block id -> no output for this unit
  bool bad = len < 1 || nt > a.max_blocks;
  if (!bad)
    for (int j = lane; j < nt; j += 64) bad |= tab[j] < 0 || tab[j] >= a.NB;
  if (__any(bad)) return;

  const int64_t tile_bytes = static_cast<int64_t>(kB) * D * E::kBytes;
  const int64_t layer_head = (static_cast<int64_t>(l) * a.NB * a.Hkv + h) * tile_bytes;
  const char* kbase = static_cast<const char*>(a.kpool) + layer_head;
  const char* vbase = static_cast<const char*>(a.vpool) + layer_head;
  const int64_t block_stride = static_cast<int64_t>(a.Hkv) * tile_bytes;

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

  for (int kt = 0; kt < nt; ++kt) {
    const int64_t boff = tab[kt] * block_stride;
    FragT kf;
    if (kt * kB + nl < len)
      kf.load(kbase + boff + (nl * D + jg * (D / 4)) * E::kBytes);
    else
      kf.zero();
    zpd::u32x4_t vv[KPL];
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
      const int key = s * RPI + vq;
      vv[s] = (kt * kB + key < len)
                  ? *reinterpret_cast<const zpd::u32x4_t*>(vbase + boff +
                                                           key * D * E::kBytes + vchunk * 16)
                  : zpd::u32x4_t{0u, 0u, 0u, 0u};
    }
    const f32x4_t sc = zpd::mma_rows<E, D>(qf, kf, f32x4_t{0.f, 0.f, 0.f, 0.f});
    const bool valid = kt * kB + nl < len;
    float p[4], alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float tm = valid ? sc[i] : -INFINITY;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) tm = fmaxf(tm, zpd::shfl_xor(tm, o));
      const float mn = fmaxf(m[i], tm);
      alpha[i] = (m[i] == -INFINITY) ? 0.f : zpd::fast_exp2((m[i] - mn) * a.sl2);
      p[i] = valid ? zpd::fast_exp2((sc[i] - mn) * a.sl2) : 0.f;
      float rs = p[i];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) rs += zpd::shfl_xor(rs, o);
      z[i] = z[i] * alpha[i] + rs;
      m[i] = mn;
    }
    // P V: lane (vchunk, vq) accumulates keys s*RPI+vq for every head g
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      const float al = __shfl(alpha[g & 3], (g >> 2) * 16, 64);
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
  }
  // sum the key sub-sets held by lanes with the same chunk, then normalise
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < VE; ++e)
      for (int o = CPR; o < 64; o <<= 1) acc[g][e] += zpd::shfl_xor(acc[g][e], o);
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    const float zg = __shfl(z[g & 3], (g >> 2) * 16, 64);
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
}

template <typename E, int D>
zp_status launch_d(const zp::DecodeGeom& g, const DecodeArgs& a, void* stream) {
  const unsigned units = static_cast<unsigned>(g.R) * g.L * g.Hkv;
  const unsigned grid = (units + 3) / 4;
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
  return ZP_OK;
}

}  // namespace

namespace zp {

zp_status launch_decode(const DecodeGeom& g, float* out, const void* q,
                        const zp_kv_pool& pool, const int32_t* tables,
                        const int32_t* seq_lens, void* stream) {
  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.kpool = pool.k;
  a.vpool = pool.v;
  a.tables = tables;
  a.seq_lens = seq_lens;
  a.R = g.R;
  a.L = g.L;
  a.Hkv = g.Hkv;
  a.Hq = g.Hq;
  a.G = g.G;
  a.NB = g.num_blocks;
  a.max_blocks = g.max_blocks;
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
