// Host side of the C ABI declared in include/zipage.h: argument checks,
// workspace layout, kernel sequencing, timing hooks and error text.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "zipage.h"
#include "zp_host.h"

namespace zp {

// ------------------------------------------------------------------ timing
namespace {
struct Pending {
  int kind;
  hipEvent_t start, stop;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_spare;
Pending g_open[ZP_KERNEL_KINDS];
bool g_is_open[ZP_KERNEL_KINDS] = {};

hipEvent_t take_event() {
  if (!g_spare.empty()) {
    hipEvent_t e = g_spare.back();
    g_spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

void timing_before(int kind, void* stream) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_timing) return;
  Pending p{kind, take_event(), take_event()};
  if (!p.start || !p.stop) return;
  (void)hipEventRecord(p.start, static_cast<hipStream_t>(stream));
  g_open[kind] = p;
  g_is_open[kind] = true;
}

void timing_after(int kind, void* stream) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_timing || !g_is_open[kind]) return;
  Pending p = g_open[kind];
  g_is_open[kind] = false;
  (void)hipEventRecord(p.stop, static_cast<hipStream_t>(stream));
  g_pending.push_back(p);
}

// ---------------------------------------------------------- common checks
namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

zp_status check_pool(const zp_kv_pool* pool) {
  if (!pool) return fail(ZP_EINVAL, "pool is NULL");
  if (!pool->k || !pool->v) return fail(ZP_EINVAL, "pool k/v pointer is NULL");
  if (!aligned16(pool->k) || !aligned16(pool->v))
    return fail(ZP_EINVAL, "pool k/v must be 16-byte aligned");
  if (pool->num_blocks <= 0 || pool->layers <= 0 || pool->kv_heads <= 0 ||
      pool->block_size <= 0 || pool->head_dim <= 0)
    return fail(ZP_EINVAL, "pool sizes must be positive");
  if (pool->dtype != ZP_F32 && pool->dtype != ZP_BF16)
    return fail(ZP_EINVAL, "pool dtype %d unknown", pool->dtype);
  if (pool->block_size != 16)
    return fail(ZP_EUNSUPPORTED, "block_size %d (the library supports 16)",
                pool->block_size);
  if (pool->head_dim != 64 && pool->head_dim != 128)
    return fail(ZP_EUNSUPPORTED, "head_dim %d (the library supports 64 and 128)",
                pool->head_dim);
  return ZP_OK;
}

float scale_log2(const zp_params* p, int d) {
  const float sc = p->sm_scale > 0.f ? p->sm_scale : 1.0f / std::sqrt(static_cast<float>(d));
  return sc * 1.4426950408889634f;
}

zp_status make_geom(const zp_kv_pool* pool, const zp_params* p,
                    const zp_batch* b, CompressGeom* g) {
  zp_status st = check_pool(pool);
  if (st != ZP_OK) return st;
  if (!p || !b) return fail(ZP_EINVAL, "params/batch is NULL");
  if (b->num_reqs < 0) return fail(ZP_EINVAL, "num_reqs < 0");
  if (p->n_max < 2) return fail(ZP_EINVAL, "n_max must be >= 2");
  // n_max * b <= n_cap <= 16384 (b = 16): larger caps are not supported, and
  // bounding n_max here keeps the products below within int range
  if (p->n_max > 1024)
    return fail(ZP_EUNSUPPORTED, "n_max %d > 1024 (n_cap is at most 16384)", p->n_max);
  if (p->q_heads <= 0 || p->q_heads % pool->kv_heads)
    return fail(ZP_EINVAL, "q_heads %d is not a positive multiple of kv_heads %d",
                p->q_heads, pool->kv_heads);
  if (p->q_dtype != pool->dtype)
    return fail(ZP_EUNSUPPORTED, "q_dtype must equal the pool dtype");
  if (p->window < 1 || p->window > p->n_max * pool->block_size)
    return fail(ZP_EINVAL, "window %d outside [1, n_max*b]", p->window);
  if (!std::isfinite(p->w_attn) || !std::isfinite(p->w_global) ||
      !std::isfinite(p->w_red) || !std::isfinite(p->sm_scale))
    return fail(ZP_EINVAL, "score weights and scale must be finite");
  if (p->flags & ~(ZP_NONCAUSAL | ZP_PROTECT_WINDOW | ZP_WINDOW_RING | ZP_UPDATE_GLOBAL |
                   ZP_SPLIT_UNITS))
    return fail(ZP_EINVAL, "unknown flags 0x%x", p->flags);
  const int k = (p->n_max - 1) * pool->block_size;
  if ((p->flags & ZP_PROTECT_WINDOW) && p->window > k)
    return fail(ZP_EINVAL, "protected window %d exceeds k = %d", p->window, k);
  if (b->max_blocks < p->n_max)
    return fail(ZP_EINVAL, "max_blocks %d < n_max %d", b->max_blocks, p->n_max);
  if (b->num_slots < 1) return fail(ZP_EINVAL, "num_slots must be >= 1");
  if (b->n_cap < p->n_max * pool->block_size)
    return fail(ZP_EINVAL, "n_cap %d < n_max*b", b->n_cap);
  if (b->n_cap > 16384) return fail(ZP_EUNSUPPORTED, "n_cap %d > 16384", b->n_cap);
  if (b->num_reqs > 0 && (!b->slot || !b->n_tokens || !b->src_table ||
                          !b->dst_table || !b->n_pinned))
    return fail(ZP_EINVAL, "batch device arrays must be non-NULL");
  const int64_t units = static_cast<int64_t>(b->num_reqs) * pool->layers * pool->kv_heads;
  if (units > (1ll << 31) - 1) return fail(ZP_EINVAL, "too many units");
  g->R = b->num_reqs;
  g->L = pool->layers;
  g->Hkv = pool->kv_heads;
  g->Hq = p->q_heads;
  g->G = p->q_heads / pool->kv_heads;
  g->d = pool->head_dim;
  g->b = pool->block_size;
  g->n_max = p->n_max;
  g->k = k;
  g->w = p->window;
  g->wG = p->window * g->G;
  g->n_cap = b->n_cap;
  g->num_blocks = pool->num_blocks;
  g->max_blocks = b->max_blocks;
  g->num_slots = b->num_slots;
  g->dtype = pool->dtype;
  g->q_dtype = p->q_dtype;
  g->flags = p->flags;
  g->w_attn = p->w_attn;
  g->w_global = p->w_global;
  g->w_red = p->w_red;
  g->scale_log2 = scale_log2(p, pool->head_dim);
  if (g->wG > 192)
    return fail(ZP_EUNSUPPORTED, "window rows w*G = %d exceed 192", g->wG);
  return ZP_OK;
}

// workspace: [0,256) error word; with ZP_SPLIT_UNITS on a bf16 pool, then
// the split-unit schedule's ticket, abort flag and group exchange slots
constexpr size_t kWsHeader = 256;

size_t workspace_for(const zp_kv_pool* pool, const zp_params* params) {
  return (pool->dtype == ZP_BF16 && (params->flags & ZP_SPLIT_UNITS)) ? split_workspace_bytes()
                                                                      : kWsHeader;
}

}  // namespace
}  // namespace zp

using namespace zp;

extern "C" {

zp_status zp_compress_workspace_bytes(const zp_kv_pool* pool,
                                      const zp_params* params, int32_t num_reqs,
                                      size_t* bytes) {
  if (!pool || !params || !bytes || num_reqs < 0)
    return fail(ZP_EINVAL, "zp_compress_workspace_bytes: bad arguments");
  if (pool->layers <= 0 || pool->kv_heads <= 0)
    return fail(ZP_EINVAL, "zp_compress_workspace_bytes: bad pool sizes");
  *bytes = workspace_for(pool, params);
  return ZP_OK;
}

zp_status zp_compress(const zp_kv_pool* pool, const zp_batch* batch,
                      const void* q_window, float* global_scores,
                      const zp_params* params, const zp_compress_out* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  CompressGeom g;
  zp_status st = make_geom(pool, params, batch, &g);
  if (st != ZP_OK) return st;
  if (!q_window || !global_scores || !out || !out->keep_idx || !out->attn)
    return fail(ZP_EINVAL, "zp_compress: q_window, global_scores, keep_idx and "
                "attn are required");
  if (!aligned16(q_window))
    return fail(ZP_EINVAL, "zp_compress: q_window must be 16-byte aligned");
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(ZP_EWORKSPACE, "zp_compress: workspace NULL or not 256-byte aligned");
  if (workspace_bytes < kWsHeader)
    return fail(ZP_EWORKSPACE, "zp_compress: workspace %zu < %zu bytes",
                workspace_bytes, kWsHeader);
  if (g.R == 0) return ZP_OK;
  int32_t* err = static_cast<int32_t*>(workspace);
  timing_before(ZP_KERNEL_COMPRESS, stream);
  if (split_eligible(g, workspace_bytes))
    st = launch_compress_split(g, *pool, *batch, q_window, global_scores, *out, workspace,
                               stream);
  else
    st = launch_compress(g, *pool, *batch, q_window, global_scores, *out, err, stream);
  timing_after(ZP_KERNEL_COMPRESS, stream);
  return st;
}

zp_status zp_update_global(float* global_scores, const zp_kv_pool* pool,
                           const zp_batch* batch, const zp_compress_out* out,
                           const zp_params* params, void* stream) {
  CompressGeom g;
  zp_status st = make_geom(pool, params, batch, &g);
  if (st != ZP_OK) return st;
  if (!global_scores || !out || !out->keep_idx || !out->attn)
    return fail(ZP_EINVAL, "zp_update_global: global_scores, keep_idx and attn "
                "are required");
  if (g.R == 0) return ZP_OK;
  timing_before(ZP_KERNEL_GLOBAL, stream);
  st = launch_global(g, global_scores, *batch, out->keep_idx, out->attn, stream);
  timing_after(ZP_KERNEL_GLOBAL, stream);
  return st;
}

zp_status zp_workspace_error(void* workspace, void* stream, int32_t* code) {
  if (!workspace || !code) return fail(ZP_EINVAL, "zp_workspace_error: bad arguments");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(ZP_EHIP, "zp_workspace_error: %s", hipGetErrorString(e));
  const int32_t zero = 0;
  e = hipMemcpyAsync(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(ZP_EHIP, "zp_workspace_error: %s", hipGetErrorString(e));
  // the kernels store ZP_EDEVICE or ZP_ESYNC; any other nonzero word is
  // reported as ZP_EDEVICE
  *code = word == 0 ? ZP_OK : word == ZP_ESYNC ? ZP_ESYNC : ZP_EDEVICE;
  return ZP_OK;
}

}  // extern "C"

namespace {

constexpr int kMaxSplits = 256;

}  // namespace

namespace zp {

size_t decode_ws_bytes(const zp_kv_pool* pool, const zp_params* params, int32_t num_reqs,
                       int32_t splits) {
  return static_cast<size_t>(num_reqs) * pool->layers * params->q_heads * splits *
         (pool->head_dim + 2) * sizeof(float);
}

// Shared checks and launch of the decode entry points.
zp_status decode_common(const char* name, float* out, const void* q, const void* k_new,
                        const void* v_new, const zp_kv_pool* pool,
                        const int32_t* block_tables, int32_t max_blocks,
                        const int32_t* seq_lens, int32_t num_reqs,
                        const zp_params* params, int32_t splits, void* workspace,
                        size_t workspace_bytes, void* stream) {
  zp_status st = check_pool(pool);
  if (st != ZP_OK) return st;
  if (!params || num_reqs < 0 || max_blocks < 1)
    return fail(ZP_EINVAL, "%s: bad arguments", name);
  if (splits < 1 || splits > kMaxSplits)
    return fail(ZP_EINVAL, "%s: splits %d outside [1, %d]", name, splits, kMaxSplits);
  if (num_reqs > 0 && (!out || !q || !block_tables || !seq_lens))
    return fail(ZP_EINVAL, "%s: NULL device array", name);
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_new) || !aligned16(v_new))
    return fail(ZP_EINVAL, "%s: out, q, k_new and v_new must be 16-byte aligned", name);
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(ZP_EINVAL, "%s: k_new and v_new go together", name);
  if (params->q_heads <= 0 || params->q_heads % pool->kv_heads)
    return fail(ZP_EINVAL, "%s: q_heads not a multiple of kv_heads", name);
  if (params->q_dtype != pool->dtype)
    return fail(ZP_EUNSUPPORTED, "%s: q_dtype must equal pool dtype", name);
  if (!std::isfinite(params->sm_scale))
    return fail(ZP_EINVAL, "%s: sm_scale must be finite", name);
  if (static_cast<int64_t>(num_reqs) * pool->layers * pool->kv_heads * splits >
      (1ll << 31) - 4)
    return fail(ZP_EINVAL, "%s: too many units", name);
  if (splits > 1) {
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
      return fail(ZP_EWORKSPACE, "%s: workspace NULL or not 256-byte aligned", name);
    if (workspace_bytes < decode_ws_bytes(pool, params, num_reqs, splits))
      return fail(ZP_EWORKSPACE, "%s: workspace %zu < %zu bytes", name, workspace_bytes,
                  decode_ws_bytes(pool, params, num_reqs, splits));
  }
  if (num_reqs == 0) return ZP_OK;
  DecodeGeom g;
  g.R = num_reqs;
  g.L = pool->layers;
  g.Hkv = pool->kv_heads;
  g.Hq = params->q_heads;
  g.G = params->q_heads / pool->kv_heads;
  g.d = pool->head_dim;
  g.b = pool->block_size;
  g.num_blocks = pool->num_blocks;
  g.max_blocks = max_blocks;
  g.dtype = pool->dtype;
  g.q_dtype = params->q_dtype;
  g.splits = splits;
  g.scale_log2 = scale_log2(params, pool->head_dim);
  DecodeIO io;
  io.out = out;
  io.q = q;
  io.tables = block_tables;
  io.seq_lens = seq_lens;
  io.k_new = k_new;
  io.v_new = v_new;
  io.part_acc = static_cast<float*>(workspace);
  io.part_mz = splits > 1 ? io.part_acc + static_cast<size_t>(num_reqs) * g.L * g.Hq *
                                              splits * g.d
                          : nullptr;
  timing_before(ZP_KERNEL_DECODE, stream);
  st = launch_decode(g, io, *pool, stream);
  timing_after(ZP_KERNEL_DECODE, stream);
  return st;
}

}  // namespace zp

extern "C" {

zp_status zp_paged_decode(float* out, const void* q, const zp_kv_pool* pool,
                          const int32_t* block_tables, int32_t max_blocks,
                          const int32_t* seq_lens, int32_t num_reqs,
                          const zp_params* params, void* stream) {
  return decode_common("zp_paged_decode", out, q, nullptr, nullptr, pool, block_tables,
                       max_blocks, seq_lens, num_reqs, params, 1, nullptr, 0, stream);
}

zp_status zp_paged_decode_append(float* out, const void* q, const void* k_new,
                                 const void* v_new, const zp_kv_pool* pool,
                                 const int32_t* block_tables, int32_t max_blocks,
                                 const int32_t* seq_lens, int32_t num_reqs,
                                 const zp_params* params, void* stream) {
  if (num_reqs > 0 && (!k_new || !v_new))
    return fail(ZP_EINVAL, "zp_paged_decode_append: k_new and v_new are required");
  return decode_common("zp_paged_decode_append", out, q, k_new, v_new, pool, block_tables,
                       max_blocks, seq_lens, num_reqs, params, 1, nullptr, 0, stream);
}

zp_status zp_decode_workspace_bytes(const zp_kv_pool* pool, const zp_params* params,
                                    int32_t num_reqs, int32_t splits, size_t* bytes) {
  if (!pool || !params || !bytes || num_reqs < 0 || splits < 1 || splits > kMaxSplits ||
      params->q_heads <= 0 || pool->layers < 1 || pool->head_dim < 1)
    return fail(ZP_EINVAL, "zp_decode_workspace_bytes: bad arguments");
  *bytes = splits > 1 ? decode_ws_bytes(pool, params, num_reqs, splits) : 0;
  return ZP_OK;
}

zp_status zp_paged_decode_split(float* out, const void* q, const void* k_new,
                                const void* v_new, const zp_kv_pool* pool,
                                const int32_t* block_tables, int32_t max_blocks,
                                const int32_t* seq_lens, int32_t num_reqs,
                                const zp_params* params, int32_t splits, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return decode_common("zp_paged_decode_split", out, q, k_new, v_new, pool, block_tables,
                       max_blocks, seq_lens, num_reqs, params, splits, workspace,
                       workspace_bytes, stream);
}

zp_status zp_redundancy_full(float* red_block, float* red_all, const zp_kv_pool* pool,
                             const zp_batch* batch, const zp_params* params,
                             void* workspace, size_t workspace_bytes, void* stream) {
  CompressGeom g;
  zp_status st = make_geom(pool, params, batch, &g);
  if (st != ZP_OK) return st;
  if (!red_block) return fail(ZP_EINVAL, "zp_redundancy_full: red_block is required");
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) ||
      workspace_bytes < kWsHeader)
    return fail(ZP_EWORKSPACE, "zp_redundancy_full: workspace missing, misaligned or small");
  if (g.R == 0) return ZP_OK;
  timing_before(ZP_KERNEL_REDUNDANCY_FULL, stream);
  st = launch_redundancy_full(g, *pool, *batch, red_block, red_all,
                              static_cast<int32_t*>(workspace), stream);
  timing_after(ZP_KERNEL_REDUNDANCY_FULL, stream);
  return st;
}

zp_status zp_capture_queries(void* q_window, const void* q, const int32_t* slot,
                             const int32_t* pos, int32_t num_reqs, int32_t layers,
                             int32_t num_slots, int32_t head_dim,
                             const zp_params* params, void* stream) {
  if (!params || num_reqs < 0 || layers < 1 || num_slots < 1)
    return fail(ZP_EINVAL, "zp_capture_queries: bad arguments");
  if (head_dim != 64 && head_dim != 128)
    return fail(ZP_EUNSUPPORTED, "zp_capture_queries: head_dim %d", head_dim);
  if (params->q_dtype != ZP_F32 && params->q_dtype != ZP_BF16)
    return fail(ZP_EINVAL, "zp_capture_queries: q_dtype %d", params->q_dtype);
  if (params->window < 1 || params->q_heads < 1)
    return fail(ZP_EINVAL, "zp_capture_queries: window and q_heads must be >= 1");
  if (num_reqs == 0) return ZP_OK;
  if (!q_window || !q || !slot || !pos)
    return fail(ZP_EINVAL, "zp_capture_queries: NULL device array");
  if (!aligned16(q_window) || !aligned16(q))
    return fail(ZP_EINVAL, "zp_capture_queries: q_window and q must be 16-byte aligned");
  const int64_t rows = static_cast<int64_t>(num_reqs) * layers;
  if (rows > (1ll << 31) - 1) return fail(ZP_EINVAL, "zp_capture_queries: too many rows");
  const int32_t row_bytes =
      params->q_heads * head_dim * (params->q_dtype == ZP_BF16 ? 2 : 4);
  timing_before(ZP_KERNEL_CAPTURE, stream);
  const zp_status st = launch_capture(q_window, q, slot, pos, num_reqs, layers,
                                      num_slots, params->window, row_bytes, stream);
  timing_after(ZP_KERNEL_CAPTURE, stream);
  return st;
}

zp_status zp_timing_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = enable != 0;
  return ZP_OK;
}

zp_status zp_timing_read(int32_t* launches, double* total_ms) {
  if (!launches || !total_ms) return fail(ZP_EINVAL, "zp_timing_read: NULL output");
  std::lock_guard<std::mutex> lk(g_tmu);
  for (int i = 0; i < ZP_KERNEL_KINDS; ++i) {
    launches[i] = 0;
    total_ms[i] = 0.0;
  }
  zp_status st = ZP_OK;
  for (const Pending& p : g_pending) {
    hipError_t e = hipEventSynchronize(p.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.start, p.stop);
    if (e != hipSuccess) {
      st = fail(ZP_EHIP, "zp_timing_read: %s", hipGetErrorString(e));
    } else {
      launches[p.kind] += 1;
      total_ms[p.kind] += ms;
    }
    g_spare.push_back(p.start);
    g_spare.push_back(p.stop);
  }
  g_pending.clear();
  return st;
}

const char* zp_version(void) { return "zipage-gfx950 0.1"; }

}  // extern "C"
