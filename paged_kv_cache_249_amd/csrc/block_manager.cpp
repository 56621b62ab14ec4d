// Host block manager of the paged KV cache (no device memory).
//
// Policy (the pages fix the mechanism, this file fixes the details):
//  * On-demand allocation from one shared free list; any free block serves
//    ("KV Cache与长上下文管理", the section on fragmentation). The free list is a
//    FIFO initialised in the caller's order; a block whose count reaches zero
//    returns to the tail.
//  * Per-block reference counts and copy-on-write on append ("PagedAttention —
//    把 KV cache 当虚拟内存页来管理", 核心要点 and 实践案例 / 案例 3): an append at
//    offset > 0 into a last block shared by others takes a fresh block, drops
//    the shared count by one and reports the (src, dst) pair to copy first.
//  * Sliding-window ring ("KV Cache与长上下文管理", the section on the second
//    problem paging solves; "PagedAttention的终极用途", part 三): with a window of
//    W blocks, opening block W+1 invalidates the oldest live block and reuses
//    its physical id for the new one; only the table row changes (front
//    dropped, id appended). An oldest block still shared by another sequence
//    cannot be overwritten: its count drops and a fresh block is taken.
//  * Swapping ("KV Cache与长上下文管理", the fourth point: a paged cache can move
//    page by page between device and host memory). The unit is a sequence's
//    live blocks. Swap-out gives each a block of a host pool (FIFO free list
//    of its own), in logical order, and reports (device, host) copy pairs; a
//    device block no one else holds returns to the device free list, a shared
//    one only loses a count. Swap-in takes device blocks from the free list
//    and reports (host, device) pairs; host blocks return to the host list.
//    A swapped-out sequence cannot append, fork or be exported.
//  * Prefix caching ("KV Cache与长上下文管理", section 二 item 2: a common prefix
//    is stored once and reused). A sequence registered from its token ids
//    shares every leading full block found under the key (previous physical
//    block or -1, the block's token ids); the rest are fresh and registered.
//    Keying on the previous block makes a match imply the whole prefix
//    matches. A block leaves the index when its count reaches zero. Not
//    offered with a ring (evicted blocks would leave stale keys).
//  * Every call is atomic; batched appends roll back through an undo log.
#include <algorithm>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

namespace {

struct Seq {
  std::deque<int32_t> table;  // live physical blocks in logical order
  int64_t tokens = 0;         // tokens appended in total
  int64_t evicted = 0;        // blocks dropped by the ring
  bool swapped = false;       // table holds host-pool block ids
};

enum class Kind : int8_t { kInPlace, kFresh, kRingReuse, kRingFresh, kCow };

// Key of a full block in the prefix index: the physical block before it in
// the sequence (-1 for the first) and the block's token ids.
struct PrefixKey {
  int32_t prev;
  std::vector<int32_t> tokens;
  bool operator==(const PrefixKey& o) const { return prev == o.prev && tokens == o.tokens; }
};

struct PrefixKeyHash {
  size_t operator()(const PrefixKey& k) const {
    // FNV-1a over the previous block id and the token ids.
    uint64_t h = 1469598103934665603ull;
    auto mix = [&h](uint32_t x) {
      for (int i = 0; i < 4; ++i) {
        h ^= (x >> (8 * i)) & 0xffu;
        h *= 1099511628211ull;
      }
    };
    mix(uint32_t(k.prev));
    for (int32_t t : k.tokens) mix(uint32_t(t));
    return size_t(h);
  }
};

struct Undo {
  int64_t seq;
  Kind kind;
  int32_t a;  // old / src block
  int32_t b;  // new / dst block
};

}  // namespace

struct pa_bm {
  int32_t num_blocks;
  int32_t block_size;
  int32_t window;
  std::deque<int32_t> free_list;
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  int32_t num_host_blocks = 0;
  std::deque<int32_t> host_free;
  std::unordered_map<PrefixKey, int32_t, PrefixKeyHash> prefix;   // key -> block
  std::unordered_map<int32_t, PrefixKey> prefix_key;               // block -> its key

  // Drop one count of device block b; at zero it returns to the free list
  // (tail) and leaves the prefix index.
  void release(int32_t b) {
    ref[b] -= 1;
    if (ref[b] == 0) {
      free_list.push_back(b);
      auto it = prefix_key.find(b);
      if (it != prefix_key.end()) {
        prefix.erase(it->second);
        prefix_key.erase(it);
      }
    }
  }

  int64_t live_tokens(const Seq& s) const { return s.tokens - int64_t(block_size) * s.evicted; }

  int32_t take_free() {
    int32_t b = free_list.front();
    free_list.pop_front();
    ref[b] = 1;
    return b;
  }

  void give_back(int32_t b) {  // exact inverse of take_free
    ref[b] = 0;
    free_list.push_front(b);
  }

  // One append; fills *u with what undoes it.
  pa_status append(int64_t id, int64_t* slot, int32_t* src, int32_t* dst, Undo* u) {
    auto it = seqs.find(id);
    if (it == seqs.end()) return pa::fail(PA_ERR_STATE, "pa_bm_append: unknown sequence %lld", (long long)id);
    Seq& s = it->second;
    if (s.swapped) return pa::fail(PA_ERR_STATE, "pa_bm_append: sequence %lld is swapped out", (long long)id);
    const int32_t offset = int32_t(s.tokens % block_size);
    *src = -1;
    *dst = -1;
    u->seq = id;
    if (offset == 0) {
      if (window > 0 && int32_t(s.table.size()) == window) {
        const int32_t oldest = s.table.front();
        if (ref[oldest] == 1) {
          s.table.pop_front();
          s.table.push_back(oldest);  // reused in place: no KV data moves
          *u = Undo{id, Kind::kRingReuse, oldest, -1};
        } else {
          if (free_list.empty())
            return pa::fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_append: no free block (ring, shared oldest)");
          s.table.pop_front();
          ref[oldest] -= 1;
          const int32_t b = take_free();
          s.table.push_back(b);
          *u = Undo{id, Kind::kRingFresh, oldest, b};
        }
        s.evicted += 1;
      } else {
        if (free_list.empty()) return pa::fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_append: no free block");
        const int32_t b = take_free();
        s.table.push_back(b);
        *u = Undo{id, Kind::kFresh, -1, b};
      }
    } else {
      const int32_t last = s.table.back();
      if (ref[last] > 1) {
        if (free_list.empty())
          return pa::fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_append: no free block for copy-on-write");
        const int32_t b = take_free();
        ref[last] -= 1;
        s.table.back() = b;
        *src = last;
        *dst = b;
        *u = Undo{id, Kind::kCow, last, b};
      } else {
        *u = Undo{id, Kind::kInPlace, -1, -1};
      }
    }
    s.tokens += 1;
    *slot = int64_t(s.table.back()) * block_size + offset;
    return PA_OK;
  }

  void undo(const Undo& u) {
    Seq& s = seqs.at(u.seq);
    s.tokens -= 1;
    switch (u.kind) {
      case Kind::kInPlace:
        break;
      case Kind::kFresh:
        s.table.pop_back();
        give_back(u.b);
        break;
      case Kind::kRingReuse:
        s.table.pop_back();
        s.table.push_front(u.a);
        s.evicted -= 1;
        break;
      case Kind::kRingFresh:
        s.table.pop_back();
        give_back(u.b);
        ref[u.a] += 1;
        s.table.push_front(u.a);
        s.evicted -= 1;
        break;
      case Kind::kCow:
        give_back(u.b);
        ref[u.a] += 1;
        s.table.back() = u.a;
        break;
    }
  }
};

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                       int32_t window_blocks, pa_bm** out) {
  if (!out) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0 || window_blocks < 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_create: num_blocks=%d block_size=%d window=%d",
                    num_blocks, block_size, window_blocks);
  if (!pa::block_size_supported(block_size))
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_bm_create: block_size %d (16, 32 or 64)", block_size);
  pa_bm* bm = new (std::nothrow) pa_bm();
  if (!bm) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_create: out of host memory");
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->window = window_blocks;
  bm->ref.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_create: free_order is not a permutation (entry %d)", i);
      }
      seen[b] = 1;
      bm->free_list.push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_blocks; ++b) bm->free_list.push_back(b);
  }
  *out = bm;
  pa::clear_error();
  return PA_OK;
}

pa_status pa_bm_destroy(pa_bm* bm) {
  delete bm;
  return PA_OK;
}

pa_status pa_bm_add_seq(pa_bm* bm, int64_t seq, int32_t prefill_tokens, int64_t* slots_out) {
  if (!bm) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq: bm is NULL");
  if (bm->seqs.count(seq)) return pa::fail(PA_ERR_STATE, "pa_bm_add_seq: sequence %lld exists", (long long)seq);
  if (prefill_tokens < 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq: negative prefill");
  if (prefill_tokens > 0 && !slots_out) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq: slots_out is NULL");
  const int32_t nb = (prefill_tokens + bm->block_size - 1) / bm->block_size;
  if (bm->window > 0 && nb > bm->window)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq: prefill needs %d blocks, window is %d", nb, bm->window);
  if (size_t(nb) > bm->free_list.size())
    return pa::fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_add_seq: needs %d blocks, %zu free", nb, bm->free_list.size());
  Seq s;
  for (int32_t i = 0; i < nb; ++i) s.table.push_back(bm->take_free());
  s.tokens = prefill_tokens;
  for (int32_t t = 0; t < prefill_tokens; ++t)
    slots_out[t] = int64_t(s.table[t / bm->block_size]) * bm->block_size + t % bm->block_size;
  bm->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

pa_status pa_bm_add_seq_prefix(pa_bm* bm, int64_t seq, const int32_t* tokens, int32_t n, int64_t* slots_out,
                               int32_t* shared_blocks) {
  if (!bm || n < 0 || (n > 0 && (!tokens || !slots_out)) || !shared_blocks)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq_prefix: bad arguments");
  if (bm->window > 0) return pa::fail(PA_ERR_UNSUPPORTED, "pa_bm_add_seq_prefix: prefix caching with a ring");
  if (bm->seqs.count(seq))
    return pa::fail(PA_ERR_STATE, "pa_bm_add_seq_prefix: sequence %lld exists", (long long)seq);
  const int32_t bs = bm->block_size;
  const int32_t nb = (n + bs - 1) / bs;
  // Leading full blocks already in the index.
  std::vector<int32_t> hits;
  PrefixKey key{-1, {}};
  for (int32_t i = 0; i < nb && (i + 1) * bs <= n; ++i) {
    key.tokens.assign(tokens + int64_t(i) * bs, tokens + int64_t(i + 1) * bs);
    auto it = bm->prefix.find(key);
    if (it == bm->prefix.end()) break;
    hits.push_back(it->second);
    key.prev = it->second;
  }
  const int32_t shared = int32_t(hits.size());
  if (size_t(nb - shared) > bm->free_list.size())
    return pa::fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_add_seq_prefix: needs %d blocks, %zu free", nb - shared,
                    bm->free_list.size());
  Seq s;
  int32_t prev = -1;
  for (int32_t i = 0; i < nb; ++i) {
    int32_t b;
    if (i < shared) {
      b = hits[i];
      bm->ref[b] += 1;
    } else {
      b = bm->take_free();
      if ((i + 1) * bs <= n) {
        PrefixKey k{prev, std::vector<int32_t>(tokens + int64_t(i) * bs, tokens + int64_t(i + 1) * bs)};
        bm->prefix_key.emplace(b, k);
        bm->prefix.emplace(std::move(k), b);
      }
    }
    s.table.push_back(b);
    prev = b;
  }
  s.tokens = n;
  for (int32_t t = 0; t < n; ++t)
    slots_out[t] = t / bs < shared ? -1 : int64_t(s.table[t / bs]) * bs + t % bs;
  bm->seqs.emplace(seq, std::move(s));
  *shared_blocks = shared;
  return PA_OK;
}

pa_status pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child) {
  if (!bm) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_fork: bm is NULL");
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "pa_bm_fork: unknown parent %lld", (long long)parent);
  if (it->second.swapped)
    return pa::fail(PA_ERR_STATE, "pa_bm_fork: parent %lld is swapped out", (long long)parent);
  if (bm->seqs.count(child)) return pa::fail(PA_ERR_STATE, "pa_bm_fork: child %lld exists", (long long)child);
  Seq c = it->second;
  for (int32_t b : c.table) bm->ref[b] += 1;
  bm->seqs.emplace(child, std::move(c));
  return PA_OK;
}

pa_status pa_bm_append(pa_bm* bm, int64_t seq, int64_t* slot_out, int32_t* copy_src, int32_t* copy_dst) {
  if (!bm || !slot_out || !copy_src || !copy_dst) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_append: NULL argument");
  Undo u;
  return bm->append(seq, slot_out, copy_src, copy_dst, &u);
}

pa_status pa_bm_append_batch(pa_bm* bm, const int64_t* seqs, int32_t n, int64_t* slots_out,
                             int32_t* pairs_out, int32_t* n_pairs) {
  if (!bm || n < 0 || (n > 0 && (!seqs || !slots_out || !pairs_out)) || !n_pairs)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_append_batch: bad arguments");
  std::vector<Undo> log;
  log.reserve(n);
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    Undo u;
    const pa_status st = bm->append(seqs[i], &slots_out[i], &src, &dst, &u);
    if (st != PA_OK) {
      for (auto r = log.rbegin(); r != log.rend(); ++r) bm->undo(*r);
      return st;
    }
    log.push_back(u);
    if (src >= 0) {
      pairs_out[2 * np] = src;
      pairs_out[2 * np + 1] = dst;
      ++np;
    }
  }
  *n_pairs = np;
  return PA_OK;
}

pa_status pa_bm_free_seq(pa_bm* bm, int64_t seq) {
  if (!bm) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_free_seq: bm is NULL");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "pa_bm_free_seq: unknown sequence %lld", (long long)seq);
  if (it->second.swapped) {
    for (int32_t hb : it->second.table) bm->host_free.push_back(hb);
  } else {
    for (int32_t b : it->second.table) bm->release(b);
  }
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_set_host_pool(pa_bm* bm, int32_t num_host_blocks, const int32_t* host_free_order) {
  if (!bm) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_set_host_pool: bm is NULL");
  if (bm->num_host_blocks > 0) return pa::fail(PA_ERR_STATE, "pa_bm_set_host_pool: host pool already set");
  if (num_host_blocks <= 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_set_host_pool: num_host_blocks=%d", num_host_blocks);
  std::deque<int32_t> order;
  if (host_free_order) {
    std::vector<char> seen(num_host_blocks, 0);
    for (int32_t i = 0; i < num_host_blocks; ++i) {
      const int32_t b = host_free_order[i];
      if (b < 0 || b >= num_host_blocks || seen[b])
        return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_set_host_pool: order is not a permutation (entry %d)", i);
      seen[b] = 1;
      order.push_back(b);
    }
  } else {
    for (int32_t b = 0; b < num_host_blocks; ++b) order.push_back(b);
  }
  bm->num_host_blocks = num_host_blocks;
  bm->host_free = std::move(order);
  return PA_OK;
}

pa_status pa_bm_swap_out(pa_bm* bm, int64_t seq, int32_t* pairs_out, int32_t cap, int32_t* n_pairs) {
  if (!bm || !n_pairs || cap < 0 || (cap > 0 && !pairs_out))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_swap_out: bad arguments");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "pa_bm_swap_out: unknown sequence %lld", (long long)seq);
  Seq& s = it->second;
  if (s.swapped) return pa::fail(PA_ERR_STATE, "pa_bm_swap_out: sequence %lld is swapped out", (long long)seq);
  if (bm->num_host_blocks == 0) return pa::fail(PA_ERR_STATE, "pa_bm_swap_out: no host pool");
  const int32_t nb = int32_t(s.table.size());
  if (cap < nb) return pa::fail(PA_ERR_OUT_OF_RANGE, "pa_bm_swap_out: cap %d < %d blocks", cap, nb);
  if (size_t(nb) > bm->host_free.size())
    return pa::fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_swap_out: needs %d host blocks, %zu free", nb,
                    bm->host_free.size());
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t b = s.table[i];
    const int32_t hb = bm->host_free.front();
    bm->host_free.pop_front();
    pairs_out[2 * i] = b;
    pairs_out[2 * i + 1] = hb;
    bm->release(b);
    s.table[i] = hb;
  }
  s.swapped = true;
  *n_pairs = nb;
  return PA_OK;
}

pa_status pa_bm_swap_in(pa_bm* bm, int64_t seq, int32_t* pairs_out, int32_t cap, int32_t* n_pairs) {
  if (!bm || !n_pairs || cap < 0 || (cap > 0 && !pairs_out))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_swap_in: bad arguments");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "pa_bm_swap_in: unknown sequence %lld", (long long)seq);
  Seq& s = it->second;
  if (!s.swapped) return pa::fail(PA_ERR_STATE, "pa_bm_swap_in: sequence %lld is resident", (long long)seq);
  const int32_t nb = int32_t(s.table.size());
  if (cap < nb) return pa::fail(PA_ERR_OUT_OF_RANGE, "pa_bm_swap_in: cap %d < %d blocks", cap, nb);
  if (size_t(nb) > bm->free_list.size())
    return pa::fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_swap_in: needs %d blocks, %zu free", nb, bm->free_list.size());
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t hb = s.table[i];
    const int32_t b = bm->take_free();
    pairs_out[2 * i] = hb;
    pairs_out[2 * i + 1] = b;
    bm->host_free.push_back(hb);
    s.table[i] = b;
  }
  s.swapped = false;
  *n_pairs = nb;
  return PA_OK;
}

pa_status pa_bm_is_swapped(const pa_bm* bm, int64_t seq, int32_t* out) {
  if (!bm || !out) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_is_swapped: NULL argument");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "pa_bm_is_swapped: unknown sequence %lld", (long long)seq);
  *out = it->second.swapped ? 1 : 0;
  return PA_OK;
}

pa_status pa_bm_host_free_list(const pa_bm* bm, int32_t* out, int32_t cap, int32_t* n) {
  if (!bm || !n || (cap > 0 && !out)) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_host_free_list: NULL argument");
  *n = int32_t(bm->host_free.size());
  if (cap < *n) return pa::fail(PA_ERR_OUT_OF_RANGE, "pa_bm_host_free_list: cap %d < %d", cap, *n);
  std::copy(bm->host_free.begin(), bm->host_free.end(), out);
  return PA_OK;
}

pa_status pa_bm_table(const pa_bm* bm, int64_t seq, int32_t* row, int32_t cap, int32_t* n_blocks,
                      int32_t* ctx_len) {
  if (!bm) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_table: bm is NULL");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "pa_bm_table: unknown sequence %lld", (long long)seq);
  const Seq& s = it->second;
  const int32_t nb = int32_t(s.table.size());
  if (n_blocks) *n_blocks = nb;
  if (ctx_len) *ctx_len = int32_t(bm->live_tokens(s));
  if (row) {
    if (cap < nb) return pa::fail(PA_ERR_OUT_OF_RANGE, "pa_bm_table: cap %d < %d blocks", cap, nb);
    std::copy(s.table.begin(), s.table.end(), row);
    std::fill(row + nb, row + cap, -1);
  }
  return PA_OK;
}

pa_status pa_bm_export(const pa_bm* bm, const int64_t* seqs, int32_t n, int32_t* tables, int32_t cap,
                       int32_t* ctx_out) {
  if (!bm || n < 0 || cap < 0 || (n > 0 && (!seqs || !tables || !ctx_out)))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_export: bad arguments");
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end())
      return pa::fail(PA_ERR_STATE, "pa_bm_export: unknown sequence %lld", (long long)seqs[i]);
    if (it->second.swapped)
      return pa::fail(PA_ERR_STATE, "pa_bm_export: sequence %lld is swapped out", (long long)seqs[i]);
    if (int32_t(it->second.table.size()) > cap)
      return pa::fail(PA_ERR_OUT_OF_RANGE, "pa_bm_export: sequence %lld holds %zu blocks > cap %d",
                      (long long)seqs[i], it->second.table.size(), cap);
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = tables + int64_t(i) * cap;
    std::copy(s.table.begin(), s.table.end(), row);
    std::fill(row + s.table.size(), row + cap, -1);
    ctx_out[i] = int32_t(bm->live_tokens(s));
  }
  return PA_OK;
}

pa_status pa_bm_ref_count(const pa_bm* bm, int32_t block, int32_t* out) {
  if (!bm || !out) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_ref_count: NULL argument");
  if (block < 0 || block >= bm->num_blocks)
    return pa::fail(PA_ERR_OUT_OF_RANGE, "pa_bm_ref_count: block %d outside [0, %d)", block, bm->num_blocks);
  *out = bm->ref[block];
  return PA_OK;
}

pa_status pa_bm_batch_shares(const pa_bm* bm, const int64_t* seqs, int32_t n, int32_t* out) {
  if (!bm || !out || n < 0 || (n > 0 && !seqs)) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_batch_shares: bad arguments");
  int32_t shares = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end())
      return pa::fail(PA_ERR_STATE, "pa_bm_batch_shares: unknown sequence %lld", (long long)seqs[i]);
    if (it->second.swapped || shares) continue;
    for (int32_t b : it->second.table) {
      if (bm->ref[b] > 1) {
        shares = 1;
        break;
      }
    }
  }
  *out = shares;
  return PA_OK;
}

pa_status pa_bm_num_free(const pa_bm* bm, int32_t* out) {
  if (!bm || !out) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_num_free: NULL argument");
  *out = int32_t(bm->free_list.size());
  return PA_OK;
}

pa_status pa_bm_free_list(const pa_bm* bm, int32_t* out, int32_t cap, int32_t* n) {
  if (!bm || !n || (cap > 0 && !out)) return pa::fail(PA_ERR_INVALID_ARG, "pa_bm_free_list: NULL argument");
  *n = int32_t(bm->free_list.size());
  if (cap < *n) return pa::fail(PA_ERR_OUT_OF_RANGE, "pa_bm_free_list: cap %d < %d", cap, *n);
  std::copy(bm->free_list.begin(), bm->free_list.end(), out);
  return PA_OK;
}

}  // extern "C"
