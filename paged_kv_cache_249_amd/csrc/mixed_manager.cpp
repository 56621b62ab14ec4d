// Host block manager of mixed-precision pages (no device memory).
//
// Pages used often stay in FP16, pages used rarely are stored as INT8
// ("PagedAttention 的技术溯源与演进脉络", §4.1 item 2, mixed-precision page
// management). Here the hot page of a sequence is its newest block, the one
// every decode step writes: each sequence owns one block of an fp16 "hot"
// pool for its whole life. Every older block is "cold", in an int8 pool with
// per-(block, head) fp16 scales. When the hot block is full and a token
// arrives, the block is demoted: quantised in one group per (block, head)
// into a fresh cold block (reported as a (hot, cold) pair for
// pa_demote_blocks), and the hot block is reused from offset 0. Cold blocks
// never change once written, so they are shared by reference count; a fork
// gives the child a copy of the parent's hot block. Free lists are FIFO in a
// caller-given order; freed blocks go to the tail. Block size 16. Every call
// is atomic.
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

namespace {

constexpr int32_t kMixedBlock = 16;

struct MSeq {
  std::vector<int32_t> cold;  // cold blocks in logical order
  int32_t hot = -1;
  int64_t tokens = 0;
};

struct MUndo {
  int64_t seq;
  int32_t demoted;  // cold block taken by the append, or -1
};

pa_status fill_order(std::deque<int32_t>* q, int32_t n, const int32_t* order, const char* what) {
  if (order) {
    std::vector<char> seen(n, 0);
    for (int32_t i = 0; i < n; ++i) {
      const int32_t b = order[i];
      if (b < 0 || b >= n || seen[b])
        return pa::fail(PA_ERR_INVALID_ARG, "pa_mbm_create: %s order is not a permutation (entry %d)", what, i);
      seen[b] = 1;
      q->push_back(b);
    }
  } else {
    for (int32_t b = 0; b < n; ++b) q->push_back(b);
  }
  return PA_OK;
}

}  // namespace

struct pa_mbm {
  int32_t num_cold;
  int32_t num_hot;
  std::deque<int32_t> cold_free;
  std::deque<int32_t> hot_free;
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, MSeq> seqs;

  pa_status append(int64_t id, int64_t* hot_slot, int32_t* src, int32_t* dst, MUndo* u) {
    auto it = seqs.find(id);
    if (it == seqs.end()) return pa::fail(PA_ERR_STATE, "pa_mbm_append: unknown sequence %lld", (long long)id);
    MSeq& s = it->second;
    *src = -1;
    *dst = -1;
    *u = MUndo{id, -1};
    if (s.tokens > 0 && s.tokens % kMixedBlock == 0) {
      if (cold_free.empty()) return pa::fail(PA_ERR_OUT_OF_BLOCKS, "pa_mbm_append: cold pool exhausted");
      const int32_t b = cold_free.front();
      cold_free.pop_front();
      ref[b] = 1;
      s.cold.push_back(b);
      *src = s.hot;
      *dst = b;
      u->demoted = b;
    }
    const int64_t off = s.tokens - int64_t(kMixedBlock) * int64_t(s.cold.size());
    s.tokens += 1;
    *hot_slot = int64_t(s.hot) * kMixedBlock + off;
    return PA_OK;
  }

  void undo(const MUndo& u) {
    MSeq& s = seqs.at(u.seq);
    s.tokens -= 1;
    if (u.demoted >= 0) {
      s.cold.pop_back();
      ref[u.demoted] = 0;
      cold_free.push_front(u.demoted);
    }
  }
};

extern "C" {

pa_status pa_mbm_create(int32_t num_cold, int32_t num_hot, const int32_t* cold_order, const int32_t* hot_order,
                        pa_mbm** out) {
  if (!out) return pa::fail(PA_ERR_INVALID_ARG, "pa_mbm_create: out is NULL");
  *out = nullptr;
  if (num_cold <= 0 || num_hot <= 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_mbm_create: num_cold=%d num_hot=%d", num_cold, num_hot);
  pa_mbm* m = new (std::nothrow) pa_mbm();
  if (!m) return pa::fail(PA_ERR_INVALID_ARG, "pa_mbm_create: out of host memory");
  m->num_cold = num_cold;
  m->num_hot = num_hot;
  m->ref.assign(num_cold, 0);
  pa_status st = fill_order(&m->cold_free, num_cold, cold_order, "cold");
  if (st == PA_OK) st = fill_order(&m->hot_free, num_hot, hot_order, "hot");
  if (st != PA_OK) {
    delete m;
    return st;
  }
  *out = m;
  return PA_OK;
}

pa_status pa_mbm_destroy(pa_mbm* m) {
  delete m;
  return PA_OK;
}

pa_status pa_mbm_add_seq(pa_mbm* m, int64_t seq, int32_t prefill_tokens, int64_t* cold_slots_out,
                         int64_t* hot_slots_out) {
  if (!m) return pa::fail(PA_ERR_INVALID_ARG, "pa_mbm_add_seq: manager is NULL");
  if (m->seqs.count(seq)) return pa::fail(PA_ERR_STATE, "pa_mbm_add_seq: sequence %lld exists", (long long)seq);
  if (prefill_tokens < 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_mbm_add_seq: negative prefill");
  if (prefill_tokens > 0 && (!cold_slots_out || !hot_slots_out))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_mbm_add_seq: slot outputs are NULL");
  const int32_t n = prefill_tokens;
  const int32_t nb = (n + kMixedBlock - 1) / kMixedBlock;
  const int32_t n_cold = nb > 0 ? nb - 1 : 0;
  if (m->hot_free.empty() || size_t(n_cold) > m->cold_free.size())
    return pa::fail(PA_ERR_OUT_OF_BLOCKS, "pa_mbm_add_seq: needs %d cold blocks (%zu free) and a hot block (%zu free)",
                    n_cold, m->cold_free.size(), m->hot_free.size());
  MSeq s;
  for (int32_t i = 0; i < n_cold; ++i) {
    const int32_t b = m->cold_free.front();
    m->cold_free.pop_front();
    m->ref[b] = 1;
    s.cold.push_back(b);
  }
  s.hot = m->hot_free.front();
  m->hot_free.pop_front();
  s.tokens = n;
  for (int32_t t = 0; t < n; ++t) {
    if (t < kMixedBlock * n_cold) {
      cold_slots_out[t] = int64_t(s.cold[t / kMixedBlock]) * kMixedBlock + t % kMixedBlock;
      hot_slots_out[t] = -1;
    } else {
      cold_slots_out[t] = -1;
      hot_slots_out[t] = int64_t(s.hot) * kMixedBlock + (t - kMixedBlock * n_cold);
    }
  }
  m->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

pa_status pa_mbm_append_batch(pa_mbm* m, const int64_t* seqs, int32_t n, int64_t* hot_slots_out,
                              int32_t* demote_pairs_out, int32_t* n_pairs) {
  if (!m || n < 0 || (n > 0 && (!seqs || !hot_slots_out || !demote_pairs_out)) || !n_pairs)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_mbm_append_batch: bad arguments");
  std::vector<MUndo> log;
  log.reserve(n);
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    MUndo u;
    const pa_status st = m->append(seqs[i], &hot_slots_out[i], &src, &dst, &u);
    if (st != PA_OK) {
      for (auto r = log.rbegin(); r != log.rend(); ++r) m->undo(*r);
      return st;
    }
    log.push_back(u);
    if (src >= 0) {
      demote_pairs_out[2 * np] = src;
      demote_pairs_out[2 * np + 1] = dst;
      ++np;
    }
  }
  *n_pairs = np;
  return PA_OK;
}

pa_status pa_mbm_fork(pa_mbm* m, int64_t parent, int64_t child, int32_t* copy_src, int32_t* copy_dst) {
  if (!m || !copy_src || !copy_dst) return pa::fail(PA_ERR_INVALID_ARG, "pa_mbm_fork: NULL argument");
  auto it = m->seqs.find(parent);
  if (it == m->seqs.end()) return pa::fail(PA_ERR_STATE, "pa_mbm_fork: unknown parent %lld", (long long)parent);
  if (m->seqs.count(child)) return pa::fail(PA_ERR_STATE, "pa_mbm_fork: child %lld exists", (long long)child);
  if (m->hot_free.empty()) return pa::fail(PA_ERR_OUT_OF_BLOCKS, "pa_mbm_fork: hot pool exhausted");
  MSeq c = it->second;
  for (int32_t b : c.cold) m->ref[b] += 1;
  c.hot = m->hot_free.front();
  m->hot_free.pop_front();
  *copy_src = it->second.hot;
  *copy_dst = c.hot;
  m->seqs.emplace(child, std::move(c));
  return PA_OK;
}

pa_status pa_mbm_free_seq(pa_mbm* m, int64_t seq) {
  if (!m) return pa::fail(PA_ERR_INVALID_ARG, "pa_mbm_free_seq: manager is NULL");
  auto it = m->seqs.find(seq);
  if (it == m->seqs.end()) return pa::fail(PA_ERR_STATE, "pa_mbm_free_seq: unknown sequence %lld", (long long)seq);
  for (int32_t b : it->second.cold) {
    m->ref[b] -= 1;
    if (m->ref[b] == 0) m->cold_free.push_back(b);
  }
  m->hot_free.push_back(it->second.hot);
  m->seqs.erase(it);
  return PA_OK;
}

pa_status pa_mbm_export(const pa_mbm* m, const int64_t* seqs, int32_t n, int32_t* cold_tables, int32_t cap,
                        int32_t* hot_out, int32_t* ctx_out) {
  if (!m || n < 0 || cap < 0 || (n > 0 && (!seqs || !cold_tables || !hot_out || !ctx_out)))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_mbm_export: bad arguments");
  for (int32_t i = 0; i < n; ++i) {
    auto it = m->seqs.find(seqs[i]);
    if (it == m->seqs.end())
      return pa::fail(PA_ERR_STATE, "pa_mbm_export: unknown sequence %lld", (long long)seqs[i]);
    if (int32_t(it->second.cold.size()) > cap)
      return pa::fail(PA_ERR_OUT_OF_RANGE, "pa_mbm_export: sequence %lld holds %zu cold blocks > cap %d",
                      (long long)seqs[i], it->second.cold.size(), cap);
  }
  for (int32_t i = 0; i < n; ++i) {
    const MSeq& s = m->seqs.find(seqs[i])->second;
    int32_t* row = cold_tables + int64_t(i) * cap;
    int32_t j = 0;
    for (; j < int32_t(s.cold.size()); ++j) row[j] = s.cold[j];
    for (; j < cap; ++j) row[j] = -1;
    hot_out[i] = s.hot;
    ctx_out[i] = int32_t(s.tokens);
  }
  return PA_OK;
}

pa_status pa_mbm_ref_count(const pa_mbm* m, int32_t cold_block, int32_t* out) {
  if (!m || !out) return pa::fail(PA_ERR_INVALID_ARG, "pa_mbm_ref_count: NULL argument");
  if (cold_block < 0 || cold_block >= m->num_cold)
    return pa::fail(PA_ERR_OUT_OF_RANGE, "pa_mbm_ref_count: block %d outside [0, %d)", cold_block, m->num_cold);
  *out = m->ref[cold_block];
  return PA_OK;
}

pa_status pa_mbm_batch_shares(const pa_mbm* m, const int64_t* seqs, int32_t n, int32_t* out) {
  if (!m || !out || n < 0 || (n > 0 && !seqs)) return pa::fail(PA_ERR_INVALID_ARG, "pa_mbm_batch_shares: bad arguments");
  int32_t shares = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = m->seqs.find(seqs[i]);
    if (it == m->seqs.end())
      return pa::fail(PA_ERR_STATE, "pa_mbm_batch_shares: unknown sequence %lld", (long long)seqs[i]);
    for (int32_t b : it->second.cold) {
      if (shares) break;
      if (m->ref[b] > 1) shares = 1;
    }
  }
  *out = shares;
  return PA_OK;
}

pa_status pa_mbm_free_lists(const pa_mbm* m, int32_t* cold_out, int32_t cold_cap, int32_t* n_cold,
                            int32_t* hot_out, int32_t hot_cap, int32_t* n_hot) {
  if (!m || !n_cold || !n_hot) return pa::fail(PA_ERR_INVALID_ARG, "pa_mbm_free_lists: NULL argument");
  *n_cold = int32_t(m->cold_free.size());
  *n_hot = int32_t(m->hot_free.size());
  if (cold_out) {
    if (cold_cap < *n_cold) return pa::fail(PA_ERR_OUT_OF_RANGE, "pa_mbm_free_lists: cold cap %d < %d", cold_cap, *n_cold);
    int32_t i = 0;
    for (int32_t b : m->cold_free) cold_out[i++] = b;
  }
  if (hot_out) {
    if (hot_cap < *n_hot) return pa::fail(PA_ERR_OUT_OF_RANGE, "pa_mbm_free_lists: hot cap %d < %d", hot_cap, *n_hot);
    int32_t i = 0;
    for (int32_t b : m->hot_free) hot_out[i++] = b;
  }
  return PA_OK;
}

}  // extern "C"
