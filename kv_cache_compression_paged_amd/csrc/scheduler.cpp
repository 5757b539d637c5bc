// Hybrid scheduling of compression and decoding on the host ([zh] §2.2,
// [de] §2, [fr] §2.B; asynchronous compression [zh] §2.1, [fr] §2.D).
//
// One step plans, for the running requests in admission order:
//   1. query slots: the first M running requests hold the M query slots;
//   2. compression: a slot holder whose cache reached N_max*b tokens (or more
//      after a prefill) and that has captured its last w queries compresses
//      this step and skips decoding; a shared-prefix compression needs free
//      target blocks, and slot-free requests are preempted to find them;
//   3. decoding: every other request appends one token, unless it holds no
//      slot and is within w tokens of the trigger (it would need its queries
//      captured: it waits for a slot). A token that opens a new block takes
//      one from the free list; when none is left the most recently admitted
//      slot-free request is preempted (its blocks return, it goes back to the
//      front of the waiting queue to be recomputed). When no slot-free
//      request is left the step runs restricted: requests that cannot get a
//      block wait and nothing is admitted;
//   4. admission, FIFO, while blocks (and, for a prompt that reaches the
//      slot threshold, a slot) are available.
// zp_sched_complete() applies the step once its GPU work is done: committed
// compressions, appended tokens, finished requests.
//
// Slot holders never exceed N_max blocks, so with num_blocks >= M*N_max
// (plus shared prefixes and targets) they always progress: the restricted
// mode cannot deadlock them.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <set>
#include <vector>

#include "zipage.h"
#include "zp_host.h"

namespace {

struct Req {
  int32_t id = 0;
  int32_t prompt = 0, gen = 0, generated = 0;
  int32_t n = 0;         // cached tokens
  int32_t seq = 0;       // sequence position of the next token
  int32_t slot = -1;
  int32_t captured = 0;  // queries captured into the slot's ring
  int32_t group = -1;
  bool running = false, finished = false;
  std::vector<int32_t> table;
};

struct Prefix {
  std::vector<int32_t> blocks;
};

}  // namespace

struct zp_sched {
  zp_sched_config cfg{};
  zp_bm* bm = nullptr;
  std::vector<Req> reqs;              // indexed by request id
  std::vector<int32_t> running;       // request ids, admission order
  std::deque<int32_t> waiting;        // request ids
  std::set<int32_t> free_slots;
  std::vector<Prefix> prefixes;
  bool pending = false;
  zp_sched_stats stats{};
  // the current plan
  zp_plan* bm_plan = nullptr;
  std::vector<int32_t> admit_id, admit_len, admit_slot, admit_table, admit_shared;
  std::vector<int32_t> new_slot;
  std::vector<int32_t> dec_id, dec_slot, dec_len, dec_pos, dec_table;
  std::vector<int32_t> cmp_id, cmp_slot, cmp_len, cmp_pos, cmp_src, cmp_dst, cmp_pinned;
  std::vector<int32_t> pre_id;
  int32_t restricted = 0;
};

namespace {

int32_t trigger(const zp_sched* s) { return s->cfg.n_max * s->cfg.block_size; }

// release every block reference of a request
void drop_blocks(zp_sched* s, Req& r) {
  if (!r.table.empty())
    zp_bm_release(s->bm, static_cast<int32_t>(r.table.size()), r.table.data());
  r.table.clear();
}

void free_slot(zp_sched* s, Req& r) {
  if (r.slot >= 0) s->free_slots.insert(r.slot);
  r.slot = -1;
  r.captured = 0;
}

// preempt the most recently admitted running request without a slot that is
// not excluded; returns its id or -1
int32_t preempt_one(zp_sched* s, const std::vector<char>& excluded) {
  for (auto it = s->running.rbegin(); it != s->running.rend(); ++it) {
    Req& v = s->reqs[*it];
    if (v.slot >= 0 || excluded[v.id]) continue;
    const int32_t id = v.id;
    drop_blocks(s, v);
    v.n = 0;
    v.running = false;
    s->running.erase(std::next(it).base());
    s->waiting.push_front(id);
    s->pre_id.push_back(id);
    s->stats.preemptions += 1;
    return id;
  }
  return -1;
}

void append_row(std::vector<int32_t>& dst, const std::vector<int32_t>& row, int32_t width) {
  for (int32_t j = 0; j < width; ++j)
    dst.push_back(j < static_cast<int32_t>(row.size()) ? row[j] : -1);
}

int32_t blocks_for(int64_t tokens, int32_t b) {
  return static_cast<int32_t>((tokens + b - 1) / b);
}

}  // namespace

extern "C" {

zp_sched* zp_sched_create(const zp_sched_config* cfg) {
  // token counts are int32: every per-request length is at most
  // max_blocks * block_size, which must stay well inside that range
  if (!cfg || cfg->num_blocks < 1 || cfg->block_size < 1 || cfg->n_max < 2 ||
      cfg->max_blocks < cfg->n_max ||
      static_cast<int64_t>(cfg->max_blocks) * cfg->block_size > (1 << 30) ||
      cfg->window < 1 || cfg->window > cfg->n_max * cfg->block_size ||
      cfg->query_slots < 1 || cfg->max_running < 1) {
    zp::set_error("zp_sched_create: bad configuration");
    return nullptr;
  }
  zp_sched* s = new (std::nothrow) zp_sched;
  if (!s) return nullptr;
  s->cfg = *cfg;
  s->bm = zp_bm_create(cfg->num_blocks);
  if (!s->bm) {
    delete s;
    return nullptr;
  }
  for (int32_t i = 0; i < cfg->query_slots; ++i) s->free_slots.insert(i);
  return s;
}

void zp_sched_destroy(zp_sched* s) {
  if (!s) return;
  if (s->bm_plan) zp_bm_abort(s->bm, s->bm_plan);
  zp_bm_destroy(s->bm);
  delete s;
}

zp_bm* zp_sched_block_manager(zp_sched* s) { return s ? s->bm : nullptr; }

zp_status zp_sched_add_prefix(zp_sched* s, int32_t blocks, int32_t* group,
                              int32_t* block_ids) {
  if (!s || blocks < 1 || blocks >= s->cfg.n_max || !group || !block_ids)
    return zp::fail(ZP_EINVAL, "zp_sched_add_prefix: bad arguments");
  if (s->pending) return zp::fail(ZP_EINVAL, "zp_sched_add_prefix: a step is pending");
  Prefix p;
  p.blocks.resize(blocks);
  const zp_status st = zp_bm_alloc(s->bm, blocks, p.blocks.data());
  if (st != ZP_OK) return st;
  std::copy(p.blocks.begin(), p.blocks.end(), block_ids);
  *group = static_cast<int32_t>(s->prefixes.size());
  s->prefixes.push_back(std::move(p));
  return ZP_OK;
}

zp_status zp_sched_submit(zp_sched* s, int32_t req_id, int32_t prompt_len,
                          int32_t gen_len, int32_t group) {
  if (!s || req_id < 0 || prompt_len < 1 || gen_len < 1)
    return zp::fail(ZP_EINVAL, "zp_sched_submit: bad arguments");
  if (static_cast<int64_t>(prompt_len) + gen_len >
      static_cast<int64_t>(s->cfg.max_blocks) * s->cfg.block_size)
    return zp::fail(ZP_EINVAL, "zp_sched_submit: prompt + generation exceed max_blocks*b");
  if (group >= static_cast<int32_t>(s->prefixes.size()) ||
      (group >= 0 && prompt_len < static_cast<int32_t>(s->prefixes[group].blocks.size()) *
                                      s->cfg.block_size))
    return zp::fail(ZP_EINVAL, "zp_sched_submit: bad prefix group");
  if (req_id < static_cast<int32_t>(s->reqs.size()) &&
      (s->reqs[req_id].running || s->reqs[req_id].prompt > 0))
    return zp::fail(ZP_EINVAL, "zp_sched_submit: request id %d already used", req_id);
  if (req_id >= static_cast<int32_t>(s->reqs.size())) s->reqs.resize(req_id + 1);
  Req& r = s->reqs[req_id];
  r = Req{};
  r.id = req_id;
  r.prompt = prompt_len;
  r.gen = gen_len;
  r.group = group < 0 ? -1 : group;
  s->waiting.push_back(req_id);
  return ZP_OK;
}

zp_status zp_sched_step(zp_sched* s, zp_sched_plan* plan) {
  if (!s || !plan) return zp::fail(ZP_EINVAL, "zp_sched_step: bad arguments");
  if (s->pending) return zp::fail(ZP_EINVAL, "zp_sched_step: previous step not completed");
  const int32_t b = s->cfg.block_size, w = s->cfg.window, M = s->cfg.query_slots;
  const int32_t nmax = s->cfg.n_max, mb = s->cfg.max_blocks, T = trigger(s);
  for (auto* v : {&s->admit_id, &s->admit_len, &s->admit_slot, &s->admit_table,
                  &s->admit_shared, &s->new_slot, &s->dec_id, &s->dec_slot, &s->dec_len,
                  &s->dec_pos, &s->dec_table, &s->cmp_id, &s->cmp_slot, &s->cmp_len,
                  &s->cmp_pos, &s->cmp_src, &s->cmp_dst, &s->cmp_pinned, &s->pre_id})
    v->clear();
  s->restricted = 0;
  std::vector<char> excluded(s->reqs.size(), 0);  // compressing or preempted

  // 1. the first M running requests hold the query slots
  for (size_t i = 0; i < s->running.size() && i < static_cast<size_t>(M); ++i) {
    Req& r = s->reqs[s->running[i]];
    if (r.slot < 0) {
      r.slot = *s->free_slots.begin();
      s->free_slots.erase(s->free_slots.begin());
      r.captured = 0;
      s->new_slot.push_back(r.slot);
    }
  }

  // 2. compressions: targets for shared prefixes may need preemptions
  std::vector<int32_t> cset;
  for (int32_t id : s->running) {
    const Req& r = s->reqs[id];
    if (r.slot >= 0 && r.n >= T && r.captured >= w) cset.push_back(id);
  }
  for (int32_t id : cset) excluded[id] = 1;
  if (!cset.empty()) {
    int64_t need = 0;
    for (int32_t id : cset) {
      const Req& r = s->reqs[id];
      int32_t sh = 0;
      while (sh < nmax - 1 && zp_bm_refcount(s->bm, r.table[sh]) > 1) ++sh;
      if (sh > 0) need += nmax - 1 - sh;
    }
    while (zp_bm_free_count(s->bm) < need && preempt_one(s, excluded) >= 0) {
    }
    if (zp_bm_free_count(s->bm) < need) {
      s->restricted = 1;       // compressions wait for blocks
      for (int32_t id : cset) excluded[id] = 0;
      cset.clear();
    }
  }
  for (int32_t id : s->pre_id) excluded[id] = 1;
  if (!cset.empty()) {
    const int32_t R = static_cast<int32_t>(cset.size());
    std::vector<int32_t> tabs, ntok;
    for (int32_t id : cset) {
      append_row(tabs, s->reqs[id].table, mb);
      ntok.push_back(s->reqs[id].n);
    }
    s->cmp_dst.assign(static_cast<size_t>(R) * nmax, -1);
    s->cmp_pinned.assign(R, 0);
    const zp_status st = zp_bm_plan_compress(s->bm, R, tabs.data(), mb, ntok.data(), nmax, b,
                                             s->cmp_dst.data(), s->cmp_pinned.data(),
                                             &s->bm_plan);
    if (st != ZP_OK) return st;
    for (int32_t id : cset) {
      const Req& r = s->reqs[id];
      s->cmp_id.push_back(id);
      s->cmp_slot.push_back(r.slot);
      s->cmp_len.push_back(r.n);
      s->cmp_pos.push_back(r.seq);
      append_row(s->cmp_src, r.table, mb);
    }
  }

  // 3. decoding, in admission order (preemptions shrink `running`, so walk
  // a copy and skip whoever was preempted meanwhile)
  std::vector<int32_t> dset;
  const std::vector<int32_t> order = s->running;
  for (const int32_t id : order) {
    if (excluded[id]) continue;
    Req& r = s->reqs[id];
    if (r.slot < 0 && r.n >= T - w) continue;   // needs a slot to go on
    if (r.slot >= 0 && r.n >= T) continue;      // window incomplete: waits
    if (r.n == static_cast<int32_t>(r.table.size()) * b) {
      while (zp_bm_free_count(s->bm) == 0) {
        const int32_t v = preempt_one(s, excluded);
        if (v < 0) break;
        excluded[v] = 1;
        dset.erase(std::remove(dset.begin(), dset.end(), v), dset.end());
        if (v == id) break;
      }
      if (excluded[id]) continue;   // preempted itself
      if (zp_bm_free_count(s->bm) == 0) {
        s->restricted = 1;
        continue;
      }
      int32_t blk;
      zp_bm_alloc(s->bm, 1, &blk);
      r.table.push_back(blk);
    }
    dset.push_back(id);
  }
  for (int32_t id : dset) {
    const Req& r = s->reqs[id];
    s->dec_id.push_back(id);
    s->dec_slot.push_back(r.slot);
    s->dec_len.push_back(r.n);
    s->dec_pos.push_back(r.seq);
    append_row(s->dec_table, r.table, mb);
  }

  // 4. admission
  while (!s->restricted && !s->waiting.empty() &&
         static_cast<int32_t>(s->running.size()) < s->cfg.max_running) {
    Req& q = s->reqs[s->waiting.front()];
    const int32_t len = q.prompt + q.generated;
    const int32_t shared = q.group >= 0 ? static_cast<int32_t>(s->prefixes[q.group].blocks.size()) : 0;
    const int32_t need = blocks_for(len, b) - shared;
    const bool gets_slot = static_cast<int32_t>(s->running.size()) < M;
    if (len >= T - w && !gets_slot) break;
    if (need > zp_bm_free_count(s->bm)) break;
    s->waiting.pop_front();
    q.table.clear();
    for (int32_t j = 0; j < shared; ++j) {
      const int32_t blk = s->prefixes[q.group].blocks[j];
      zp_bm_incref(s->bm, blk);
      q.table.push_back(blk);
    }
    const size_t base = q.table.size();
    q.table.resize(base + need);
    if (need > 0) zp_bm_alloc(s->bm, need, q.table.data() + base);
    q.n = len;
    q.seq = len;
    q.running = true;
    s->running.push_back(q.id);
    if (gets_slot) {
      q.slot = *s->free_slots.begin();
      s->free_slots.erase(s->free_slots.begin());
      q.captured = std::min(w, len);   // the prompt's queries fill the ring
      s->new_slot.push_back(q.slot);
    } else {
      q.slot = -1;
      q.captured = 0;
    }
    s->admit_id.push_back(q.id);
    s->admit_len.push_back(len);
    s->admit_slot.push_back(q.slot);
    s->admit_shared.push_back(shared * b);
    append_row(s->admit_table, q.table, mb);
    s->stats.admitted += 1;
  }

  s->stats.steps += 1;
  s->stats.restricted_steps += s->restricted;
  s->pending = true;
  plan->restricted = s->restricted;
  plan->max_blocks = mb;
  plan->num_admit = static_cast<int32_t>(s->admit_id.size());
  plan->admit_id = s->admit_id.data();
  plan->admit_len = s->admit_len.data();
  plan->admit_slot = s->admit_slot.data();
  plan->admit_table = s->admit_table.data();
  plan->admit_shared = s->admit_shared.data();
  plan->num_new_slots = static_cast<int32_t>(s->new_slot.size());
  plan->new_slot = s->new_slot.data();
  plan->num_decode = static_cast<int32_t>(s->dec_id.size());
  plan->decode_id = s->dec_id.data();
  plan->decode_slot = s->dec_slot.data();
  plan->decode_len = s->dec_len.data();
  plan->decode_pos = s->dec_pos.data();
  plan->decode_table = s->dec_table.data();
  plan->num_compress = static_cast<int32_t>(s->cmp_id.size());
  plan->compress_id = s->cmp_id.data();
  plan->compress_slot = s->cmp_slot.data();
  plan->compress_len = s->cmp_len.data();
  plan->compress_pos = s->cmp_pos.data();
  plan->compress_src = s->cmp_src.data();
  plan->compress_dst = s->cmp_dst.data();
  plan->compress_pinned = s->cmp_pinned.data();
  plan->num_preempt = static_cast<int32_t>(s->pre_id.size());
  plan->preempt_id = s->pre_id.data();
  return ZP_OK;
}

zp_status zp_sched_complete(zp_sched* s) {
  if (!s || !s->pending) return zp::fail(ZP_EINVAL, "zp_sched_complete: no pending step");
  const int32_t nmax = s->cfg.n_max, b = s->cfg.block_size;
  if (s->bm_plan) {
    zp_bm_commit(s->bm, s->bm_plan);
    s->bm_plan = nullptr;
    for (size_t i = 0; i < s->cmp_id.size(); ++i) {
      Req& r = s->reqs[s->cmp_id[i]];
      r.table.assign(s->cmp_dst.begin() + i * nmax, s->cmp_dst.begin() + (i + 1) * nmax);
      r.n = (nmax - 1) * b;
      s->stats.compressions += 1;
    }
  }
  for (int32_t id : s->dec_id) {
    Req& r = s->reqs[id];
    r.n += 1;
    r.seq += 1;
    r.generated += 1;
    if (r.slot >= 0) r.captured += 1;
    s->stats.tokens += 1;
    if (r.generated >= r.gen) {
      drop_blocks(s, r);
      free_slot(s, r);
      r.running = false;
      r.finished = true;
      s->running.erase(std::find(s->running.begin(), s->running.end(), id));
      s->stats.finished += 1;
    }
  }
  s->pending = false;
  return ZP_OK;
}

zp_status zp_sched_get_stats(const zp_sched* s, zp_sched_stats* st) {
  if (!s || !st) return zp::fail(ZP_EINVAL, "zp_sched_get_stats: bad arguments");
  *st = s->stats;
  st->running = static_cast<int32_t>(s->running.size());
  st->waiting = static_cast<int32_t>(s->waiting.size());
  st->free_blocks = zp_bm_free_count(s->bm);
  return ZP_OK;
}

}  // extern "C"
