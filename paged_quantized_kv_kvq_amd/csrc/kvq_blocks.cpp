// Host block manager: free-block stack, per-block counts, per-sequence block
// tables, append with copy on write, rollback.
//
// "spark_runtime/kv_cache.rs", PagedKvCache (free_blocks, block_ref_counts);
// "combs_models/kv.rs", PageAllocator (a stack of free ids, block 0 handed out
// first), ensure_pages, popn, reset.  Plain host C++: no HIP calls.
//
// Every host allocation an entry point needs is made before the first change
// to the manager's state, so a std::bad_alloc leaves that state as it was and
// comes back as KVQ_ERR_HOST_MEMORY; no exception crosses the C interface.
#include <algorithm>
#include <cstdint>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "kvq_blocks.h"

struct kvq_blocks {
  struct Seq {
    bool live = false;
    uint32_t len = 0;
    std::vector<uint32_t> table;
  };
  uint32_t num_blocks = 0, block_size = 0;
  std::vector<uint32_t> free;   // top of the stack = back
  std::vector<uint32_t> count;  // per block
  std::vector<Seq> seqs;
  std::mutex mu;

  void reset() {
    free.resize(num_blocks);
    for (uint32_t i = 0; i < num_blocks; ++i) free[i] = num_blocks - 1 - i;  // block 0 on top
    count.assign(num_blocks, 0u);
    seqs.clear();
  }
  uint32_t take() {
    const uint32_t b = free.back();
    free.pop_back();
    count[b] = 1;
    return b;
  }
  void release(uint32_t b) {
    if (--count[b] == 0) free.push_back(b);
  }
  Seq* seq(uint32_t id) { return id < seqs.size() && seqs[id].live ? &seqs[id] : nullptr; }
  uint32_t new_id() {
    for (uint32_t i = 0; i < seqs.size(); ++i)
      if (!seqs[i].live) return i;
    seqs.emplace_back();
    return uint32_t(seqs.size() - 1);
  }
  uint64_t pages_for(uint64_t len) const { return (len + block_size - 1) / block_size; }
};

namespace {
constexpr uint32_t kMaxId = 0x7FFFFFFFu;

template <class F>
int guarded(F&& f) {
  try {
    return f();
  } catch (const std::bad_alloc&) {
    return KVQ_ERR_HOST_MEMORY;
  }
}
}  // namespace

extern "C" {

int kvq_blocks_create(uint32_t num_blocks, uint32_t block_size, kvq_blocks** out) {
  if (!out || num_blocks == 0 || num_blocks > kMaxId || block_size == 0) return KVQ_ERR_INVALID_ARG;
  kvq_blocks* bm = new (std::nothrow) kvq_blocks;
  if (!bm) return KVQ_ERR_HOST_MEMORY;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  const int st = guarded([&] {
    bm->reset();
    return int(KVQ_OK);
  });
  if (st != KVQ_OK) {
    delete bm;
    return st;
  }
  *out = bm;
  return KVQ_OK;
}

void kvq_blocks_destroy(kvq_blocks* bm) { delete bm; }

int kvq_blocks_reset(kvq_blocks* bm) {
  if (!bm) return KVQ_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(bm->mu);
  bm->reset();  // the free stack and the counts keep their size: nothing is allocated
  return KVQ_OK;
}

int kvq_blocks_num_free(kvq_blocks* bm, uint32_t* num_free) {
  if (!bm || !num_free) return KVQ_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(bm->mu);
  *num_free = uint32_t(bm->free.size());
  return KVQ_OK;
}

int kvq_blocks_ref_count(kvq_blocks* bm, uint32_t block, uint32_t* count) {
  if (!bm || !count) return KVQ_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(bm->mu);
  if (block >= bm->num_blocks) return KVQ_ERR_INVALID_ARG;
  *count = bm->count[block];
  return KVQ_OK;
}

int kvq_blocks_seq_new(kvq_blocks* bm, uint32_t* seq) {
  if (!bm || !seq) return KVQ_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(bm->mu);
  return guarded([&] {
    const uint32_t id = bm->new_id();  // the one allocation, made before any change
    bm->seqs[id] = kvq_blocks::Seq();
    bm->seqs[id].live = true;
    *seq = id;
    return int(KVQ_OK);
  });
}

int kvq_blocks_seq_fork(kvq_blocks* bm, uint32_t parent, uint32_t* child) {
  if (!bm || !child) return KVQ_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(bm->mu);
  if (!bm->seq(parent)) return KVQ_ERR_INVALID_ARG;
  return guarded([&] {
    kvq_blocks::Seq p = bm->seqs[parent];  // both allocations come before any count changes
    const uint32_t id = bm->new_id();
    for (uint32_t b : p.table) ++bm->count[b];
    bm->seqs[id] = std::move(p);
    *child = id;
    return int(KVQ_OK);
  });
}

int kvq_blocks_seq_free(kvq_blocks* bm, uint32_t seq) {
  if (!bm) return KVQ_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(bm->mu);
  kvq_blocks::Seq* s = bm->seq(seq);
  if (!s) return KVQ_ERR_INVALID_ARG;
  for (auto it = s->table.rbegin(); it != s->table.rend(); ++it) bm->release(*it);
  *s = kvq_blocks::Seq();
  return KVQ_OK;
}

int kvq_blocks_seq_len(kvq_blocks* bm, uint32_t seq, uint32_t* len, uint32_t* num_blocks) {
  if (!bm || !len || !num_blocks) return KVQ_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(bm->mu);
  const kvq_blocks::Seq* s = bm->seq(seq);
  if (!s) return KVQ_ERR_INVALID_ARG;
  *len = s->len;
  *num_blocks = uint32_t(s->table.size());
  return KVQ_OK;
}

int kvq_blocks_append(kvq_blocks* bm, uint32_t seq, uint32_t n, int64_t* slots, int32_t* cow_src,
                      int32_t* cow_dst) {
  if (!bm || !cow_src || !cow_dst || (n && !slots)) return KVQ_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(bm->mu);
  kvq_blocks::Seq* s = bm->seq(seq);
  if (!s || uint64_t(s->len) + n > kMaxId) return KVQ_ERR_INVALID_ARG;
  const uint32_t bs = bm->block_size;
  // the last block is written into when it is partly filled; shared, it is
  // copied to a fresh block first
  const bool cow = n > 0 && s->len % bs != 0 && bm->count[s->table.back()] > 1;
  const uint64_t grow = bm->pages_for(uint64_t(s->len) + n) - s->table.size();
  if (grow + (cow ? 1 : 0) > bm->free.size()) return KVQ_ERR_EXHAUSTED;
  const int st = guarded([&] {
    s->table.reserve(s->table.size() + grow);  // the pushes below then cannot throw
    return int(KVQ_OK);
  });
  if (st != KVQ_OK) return st;
  *cow_src = *cow_dst = -1;
  if (cow) {
    const uint32_t old = s->table.back();
    const uint32_t fresh = bm->take();
    bm->release(old);  // still held by the other owners
    s->table.back() = fresh;
    *cow_src = int32_t(old);
    *cow_dst = int32_t(fresh);
  }
  for (uint64_t i = 0; i < grow; ++i) s->table.push_back(bm->take());
  for (uint32_t i = 0; i < n; ++i) {
    const uint32_t p = s->len + i;
    slots[i] = int64_t(s->table[p / bs]) * bs + p % bs;
  }
  s->len += n;
  return KVQ_OK;
}

int kvq_blocks_append_many(kvq_blocks* bm, const uint32_t* seqs, const uint32_t* counts, uint32_t num_seqs,
                           int64_t* slots, int32_t* cow) {
  if (!bm || (num_seqs && (!seqs || !counts || !cow))) return KVQ_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(bm->mu);
  const uint32_t bs = bm->block_size;
  uint64_t need = 0, total = 0;
  std::vector<uint32_t> ids;
  const int st = guarded([&] {
    ids.assign(seqs, seqs + num_seqs);
    return int(KVQ_OK);
  });
  if (st != KVQ_OK) return st;
  std::sort(ids.begin(), ids.end());
  if (std::adjacent_find(ids.begin(), ids.end()) != ids.end()) return KVQ_ERR_INVALID_ARG;
  for (uint32_t i = 0; i < num_seqs; ++i) {
    const kvq_blocks::Seq* s = bm->seq(seqs[i]);
    if (!s || uint64_t(s->len) + counts[i] > kMaxId) return KVQ_ERR_INVALID_ARG;
    const bool shared = counts[i] > 0 && s->len % bs != 0 && bm->count[s->table.back()] > 1;
    need += bm->pages_for(uint64_t(s->len) + counts[i]) - s->table.size() + (shared ? 1 : 0);
    total += counts[i];
  }
  if (total && !slots) return KVQ_ERR_INVALID_ARG;
  if (need > bm->free.size()) return KVQ_ERR_EXHAUSTED;
  // every table gets its room first; extra capacity alone changes no state
  const int room = guarded([&] {
    for (uint32_t i = 0; i < num_seqs; ++i) {
      kvq_blocks::Seq* s = bm->seq(seqs[i]);
      s->table.reserve(bm->pages_for(uint64_t(s->len) + counts[i]));
    }
    return int(KVQ_OK);
  });
  if (room != KVQ_OK) return room;
  uint64_t o = 0;
  for (uint32_t i = 0; i < num_seqs; ++i) {
    kvq_blocks::Seq* s = bm->seq(seqs[i]);
    const uint32_t n = counts[i];
    cow[2 * i] = cow[2 * i + 1] = -1;
    if (n > 0 && s->len % bs != 0 && bm->count[s->table.back()] > 1) {
      const uint32_t old = s->table.back();
      const uint32_t fresh = bm->take();
      bm->release(old);
      s->table.back() = fresh;
      cow[2 * i] = int32_t(old);
      cow[2 * i + 1] = int32_t(fresh);
    }
    const uint64_t grow = bm->pages_for(uint64_t(s->len) + n) - s->table.size();
    for (uint64_t k = 0; k < grow; ++k) s->table.push_back(bm->take());
    for (uint32_t k = 0; k < n; ++k) {
      const uint32_t p = s->len + k;
      slots[o++] = int64_t(s->table[p / bs]) * bs + p % bs;
    }
    s->len += n;
  }
  return KVQ_OK;
}

int kvq_blocks_popn(kvq_blocks* bm, uint32_t seq, uint32_t n, uint32_t* popped) {
  if (!bm || !popped) return KVQ_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(bm->mu);
  kvq_blocks::Seq* s = bm->seq(seq);
  if (!s) return KVQ_ERR_INVALID_ARG;
  const uint32_t k = std::min(n, s->len);
  s->len -= k;
  const uint64_t keep = bm->pages_for(s->len);
  while (s->table.size() > keep) {
    bm->release(s->table.back());
    s->table.pop_back();
  }
  *popped = k;
  return KVQ_OK;
}

int kvq_blocks_table(kvq_blocks* bm, const uint32_t* seqs, uint32_t num_seqs, uint32_t max_blocks_per_seq,
                     int32_t* block_tables, int32_t* seq_lens) {
  if (!bm || (num_seqs && (!seqs || !block_tables || !seq_lens))) return KVQ_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(bm->mu);
  for (uint32_t i = 0; i < num_seqs; ++i) {
    const kvq_blocks::Seq* s = bm->seq(seqs[i]);
    if (!s || s->table.size() > max_blocks_per_seq) return KVQ_ERR_INVALID_ARG;
  }
  for (uint32_t i = 0; i < num_seqs; ++i) {
    const kvq_blocks::Seq* s = bm->seq(seqs[i]);
    int32_t* row = block_tables + uint64_t(i) * max_blocks_per_seq;
    std::copy(s->table.begin(), s->table.end(), row);  // ids < 2^31: the same bits as int32
    std::fill(row + s->table.size(), row + max_blocks_per_seq, -1);
    seq_lens[i] = int32_t(s->len);
  }
  return KVQ_OK;
}

}  // extern "C"
