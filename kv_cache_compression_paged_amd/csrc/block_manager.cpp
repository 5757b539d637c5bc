// Host-side block bookkeeping for compressed paged KV caches: a LIFO free
// list, per-block reference counts and the plan/commit of one compression
// call. Pure C++; no GPU calls, so it can be exercised on any host.
//
// Pages: requests hold blocks and return them when done ([zh] §2, [es] §2);
// a compression triggers at N_max full blocks and keeps (N_max-1)*b tokens
// ([zh] §2.1); blocks of a shared prefix (reference count above one) are
// never moved, compressed rows go to freshly allocated target blocks
// ([zh] §2.2, [de] §2, [fr] §2.C).
#include <cstdint>
#include <new>
#include <vector>

#include "zipage.h"
#include "zp_host.h"

struct zp_bm {
  std::vector<int32_t> refcount;
  std::vector<int32_t> stack;   // top = back()
};

struct zp_plan {
  std::vector<int32_t> popped;  // targets, in pop order
  std::vector<int32_t> freed;   // blocks to push at commit, in push order
  zp_bm* owner = nullptr;
};

extern "C" {

zp_bm* zp_bm_create(int32_t num_blocks) {
  if (num_blocks <= 0) {
    zp::set_error("zp_bm_create: num_blocks must be positive");
    return nullptr;
  }
  zp_bm* bm = new (std::nothrow) zp_bm;
  if (!bm) return nullptr;
  try {
    bm->refcount.assign(num_blocks, 0);
    bm->stack.resize(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) bm->stack[i] = num_blocks - 1 - i;
  } catch (...) {
    delete bm;
    zp::set_error("zp_bm_create: out of host memory");
    return nullptr;
  }
  return bm;
}

void zp_bm_destroy(zp_bm* bm) { delete bm; }

zp_status zp_bm_alloc(zp_bm* bm, int32_t n, int32_t* ids) {
  if (!bm || n < 0 || (n > 0 && !ids))
    return zp::fail(ZP_EINVAL, "zp_bm_alloc: bad arguments");
  if (static_cast<size_t>(n) > bm->stack.size())
    return zp::fail(ZP_ENOSPACE, "zp_bm_alloc: free list exhausted");
  for (int32_t i = 0; i < n; ++i) {
    int32_t id = bm->stack.back();
    bm->stack.pop_back();
    bm->refcount[id] = 1;
    ids[i] = id;
  }
  return ZP_OK;
}

zp_status zp_bm_incref(zp_bm* bm, int32_t id) {
  if (!bm || id < 0 || id >= static_cast<int32_t>(bm->refcount.size()))
    return zp::fail(ZP_EINVAL, "zp_bm_incref: bad block id");
  if (bm->refcount[id] < 1)
    return zp::fail(ZP_EINVAL, "zp_bm_incref: block is free");
  bm->refcount[id] += 1;
  return ZP_OK;
}

zp_status zp_bm_release(zp_bm* bm, int32_t n, const int32_t* ids) {
  if (!bm || n < 0 || (n > 0 && !ids))
    return zp::fail(ZP_EINVAL, "zp_bm_release: bad arguments");
  const int32_t nb = static_cast<int32_t>(bm->refcount.size());
  // check everything first so an error changes nothing
  std::vector<int32_t> drop(nb, 0);
  for (int32_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= nb)
      return zp::fail(ZP_EINVAL, "zp_bm_release: bad block id");
    if (++drop[ids[i]] > bm->refcount[ids[i]])
      return zp::fail(ZP_EINVAL, "zp_bm_release: block released too often");
  }
  for (int32_t i = 0; i < n; ++i) {
    if (--bm->refcount[ids[i]] == 0) bm->stack.push_back(ids[i]);
  }
  return ZP_OK;
}

int32_t zp_bm_free_count(const zp_bm* bm) {
  return bm ? static_cast<int32_t>(bm->stack.size()) : -1;
}

int32_t zp_bm_refcount(const zp_bm* bm, int32_t id) {
  if (!bm || id < 0 || id >= static_cast<int32_t>(bm->refcount.size())) return -1;
  return bm->refcount[id];
}

int32_t zp_bm_free_list(const zp_bm* bm, int32_t* ids, int32_t cap) {
  if (!bm) return -1;
  const int32_t n = static_cast<int32_t>(bm->stack.size());
  for (int32_t i = 0; i < n && i < cap && ids; ++i) ids[i] = bm->stack[i];
  return n;
}

zp_status zp_bm_plan_compress(zp_bm* bm, int32_t num_reqs,
                              const int32_t* host_tables, int32_t max_blocks,
                              const int32_t* n_tokens, int32_t n_max,
                              int32_t block_size, int32_t* dst_tables,
                              int32_t* n_pinned, zp_plan** plan) {
  if (!bm || num_reqs < 0 || max_blocks < 1 || n_max < 2 || block_size < 1 ||
      n_max > max_blocks || !plan || (num_reqs > 0 && (!host_tables ||
      !n_tokens || !dst_tables || !n_pinned)))
    return zp::fail(ZP_EINVAL, "zp_bm_plan_compress: bad arguments");
  *plan = nullptr;
  const int32_t nb = static_cast<int32_t>(bm->refcount.size());
  std::vector<int32_t> shared(num_reqs);
  std::vector<char> mark(nb, 0);
  int64_t need = 0;
  for (int32_t r = 0; r < num_reqs; ++r) {
    const int64_t n = n_tokens[r];
    const int64_t held = (n + block_size - 1) / block_size;
    if (n < static_cast<int64_t>(n_max) * block_size || held > max_blocks)
      return zp::fail(ZP_EINVAL, "zp_bm_plan_compress: request %d holds %lld "
                      "tokens, outside [n_max*b, max_blocks*b]", r,
                      static_cast<long long>(n));
    const int32_t* t = host_tables + static_cast<int64_t>(r) * max_blocks;
    for (int64_t j = 0; j < held; ++j)
      if (t[j] < 0 || t[j] >= nb)
        return zp::fail(ZP_EINVAL, "zp_bm_plan_compress: request %d block "
                        "%lld has id %d out of range", r,
                        static_cast<long long>(j), t[j]);
    int32_t s = 0;
    while (s < n_max - 1 && bm->refcount[t[s]] > 1) ++s;
    // every block past the shared run is written in place, becomes the tail
    // or is freed: it must belong to this request alone, once
    for (int64_t j = s; j < held; ++j) {
      if (bm->refcount[t[j]] != 1)
        return zp::fail(ZP_EINVAL, "zp_bm_plan_compress: request %d block %lld "
                        "(id %d) has refcount %d; blocks after the shared "
                        "prefix must be held by one request", r,
                        static_cast<long long>(j), t[j], bm->refcount[t[j]]);
      if (mark[t[j]])
        return zp::fail(ZP_EINVAL, "zp_bm_plan_compress: block id %d appears "
                        "twice among the private blocks of the call", t[j]);
      mark[t[j]] = 1;
    }
    shared[r] = s;
    if (s > 0) need += n_max - 1 - s;
  }
  if (need > static_cast<int64_t>(bm->stack.size()))
    return zp::fail(ZP_ENOSPACE, "zp_bm_plan_compress: %lld targets needed, "
                    "%zu free", static_cast<long long>(need), bm->stack.size());
  zp_plan* p = new (std::nothrow) zp_plan;
  if (!p) return zp::fail(ZP_EINVAL, "zp_bm_plan_compress: out of host memory");
  p->owner = bm;
  for (int32_t r = 0; r < num_reqs; ++r) {
    const int32_t* t = host_tables + static_cast<int64_t>(r) * max_blocks;
    int32_t* dst = dst_tables + static_cast<int64_t>(r) * n_max;
    const int64_t held = (static_cast<int64_t>(n_tokens[r]) + block_size - 1) /
                         block_size;
    const int32_t s = shared[r];
    n_pinned[r] = s;
    if (s == 0) {
      for (int32_t j = 0; j < n_max; ++j) dst[j] = t[j];
    } else {
      for (int32_t j = 0; j < s; ++j) dst[j] = t[j];
      for (int32_t j = s; j < n_max - 1; ++j) {
        const int32_t id = bm->stack.back();
        bm->stack.pop_back();
        p->popped.push_back(id);
        dst[j] = id;
      }
      dst[n_max - 1] = t[n_max - 1];
      for (int32_t j = s; j < n_max - 1; ++j) p->freed.push_back(t[j]);
    }
    for (int64_t j = n_max; j < held; ++j) p->freed.push_back(t[j]);
  }
  *plan = p;
  return ZP_OK;
}

zp_status zp_bm_commit(zp_bm* bm, zp_plan* plan) {
  if (!bm || !plan || plan->owner != bm)
    return zp::fail(ZP_EINVAL, "zp_bm_commit: plan does not belong to manager");
  for (int32_t id : plan->popped) bm->refcount[id] = 1;
  for (int32_t id : plan->freed) {
    bm->refcount[id] = 0;
    bm->stack.push_back(id);
  }
  delete plan;
  return ZP_OK;
}

zp_status zp_bm_abort(zp_bm* bm, zp_plan* plan) {
  if (!bm || !plan || plan->owner != bm)
    return zp::fail(ZP_EINVAL, "zp_bm_abort: plan does not belong to manager");
  for (auto it = plan->popped.rbegin(); it != plan->popped.rend(); ++it)
    bm->stack.push_back(*it);
  delete plan;
  return ZP_OK;
}

int32_t zp_plan_freed(const zp_plan* plan, int32_t* ids, int32_t cap) {
  if (!plan) return -1;
  const int32_t n = static_cast<int32_t>(plan->freed.size());
  for (int32_t i = 0; i < n && i < cap && ids; ++i) ids[i] = plan->freed[i];
  return n;
}

int32_t zp_plan_targets(const zp_plan* plan, int32_t* ids, int32_t cap) {
  if (!plan) return -1;
  const int32_t n = static_cast<int32_t>(plan->popped.size());
  for (int32_t i = 0; i < n && i < cap && ids; ++i) ids[i] = plan->popped[i];
  return n;
}

}  // extern "C"
