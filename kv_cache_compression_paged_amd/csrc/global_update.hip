// Global-score update ([zh] §2.1 historical attention carried across
// compressions): after a unit's compaction its global row follows its tokens,
// g'_t = g_{keep[t]} + attn_{keep[t]} for the k kept positions and zero for
// the freed tail [k, n_cap).
//
// One workgroup per unit; the row is staged in LDS before it is rewritten in
// place, so reads never see a partly updated row.
#include <hip/hip_runtime.h>

#include "zp_device.h"
#include "zp_host.h"

namespace {

constexpr int kThreads = 256;
constexpr int kB = 16;

struct GlobalArgs {
  float* glob;
  const int32_t* keep;
  const float* attn;
  const int32_t* slot;
  const int32_t* n_tokens;
  int32_t R, L, Hkv, n_cap, num_slots, n_max, k;
};

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
  // two requests naming one slot would rewrite one row together: skip both
  for (int j = threadIdx.x; j < a.R; j += kThreads) bad |= j != r && a.slot[j] == slot;
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

zp_status launch_global(const CompressGeom& g, float* global_scores,
                        const zp_batch& batch, const int32_t* keep,
                        const float* attn, void* stream) {
  GlobalArgs a;
  a.glob = global_scores;
  a.keep = keep;
  a.attn = attn;
  a.slot = batch.slot;
  a.n_tokens = batch.n_tokens;
  a.R = g.R;
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
