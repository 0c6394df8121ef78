// Host block manager: free pool, reference counts, fork, copy-on-write, block tables.
//
// Behaviour (see the policy block in pa.h):
//  * "Taming the Tail", "How the Architecture Works": logical blocks of a sequence map through
//    a block table to physical blocks anywhere in the pool; a full current block means a new
//    block from the free block pool.
//  * "vLLM PagedAttention" (tinycto), "1. Underlying Mechanism": with B = 16 the 17th token
//    takes a new block on the fly; forked children share the parent's blocks; copy-on-write
//    gives a writer its own copy.
//  * KV-cache chapter, "PagedAttention: borrowing virtual memory" and answer A6: per-block
//    reference counts; a block is free again only at count zero; a writer into a shared block
//    first receives a private copy.
//
// The free pool is a ring buffer of capacity num_blocks (a block is in it at most once), so
// allocation and release are O(1).  Every mutating call validates and sizes its work in a
// dry run first, so a failing call changes nothing.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <functional>
#include <map>
#include <new>
#include <queue>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa.h"
#include "pa_status.h"

namespace {

struct Seq {
  std::vector<int32_t> blocks;  // physical ids in logical order
  int32_t n = 0;                // tokens held
  uint64_t stamp = 0;           // the append call that last named it (repeat detection)
};

// Prefix-cache tree node: one full block of B tokens, keyed by those token ids under its
// parent.  Nodes live in a vector indexed by their id and are never reused; `live` is false
// once evicted.
using TokenKey = std::vector<int32_t>;
struct CacheNode {
  int32_t block = -1;
  TokenKey key;
  int64_t parent = -1;                    // -1: a child of the root
  std::map<TokenKey, int64_t> children;   // token ids -> node id
  int64_t last_use = 0;
  bool live = true;
};

}  // namespace

struct pa_bm {
  int32_t num_blocks = 0;
  int32_t B = 0;
  std::vector<int32_t> ref;   // per-block reference count
  std::vector<int32_t> ring;  // FIFO free pool
  int32_t head = 0;           // index of the front of the pool in `ring`
  int32_t nfree = 0;
  std::unordered_map<int64_t, Seq> seqs;
  std::unordered_map<int64_t, int32_t> swapped;  // swapped-out sequence -> its length
  int64_t forks = 0;
  int64_t cow_copies = 0;
  int64_t swap_outs = 0;
  int64_t swap_ins = 0;
  std::vector<CacheNode> nodes;           // prefix-cache tree
  std::map<TokenKey, int64_t> root;
  std::vector<int64_t> node_of_block;     // live tree node holding a block, or -1
  // Eviction candidates (last use, node id), smallest first.  Every node that is evictable
  // (a live leaf only the tree references) has an entry with its current last use; entries
  // that no longer match are skipped when popped.
  std::priority_queue<std::pair<int64_t, int64_t>, std::vector<std::pair<int64_t, int64_t>>,
                      std::greater<std::pair<int64_t, int64_t>>> cand;
  int64_t tick = 0;
  // Per-call scratch of the append calls, kept so a decode step allocates nothing once the
  // vectors have grown to the batch size.
  uint64_t epoch = 0;
  std::vector<Seq*> batch;
  // The ids `batch` was resolved from, valid while no sequence has been erased since (erasing
  // is the only way an element's address in `seqs` changes): a serving loop names the same
  // batch step after step, and then no id is looked up again.
  std::vector<int64_t> batch_ids;
  bool batch_valid = false;
  uint64_t seq_erasures = 0;
  uint64_t batch_erasures = 0;
  std::vector<char> cow;
  std::unordered_map<int32_t, int32_t> dec;  // shared block -> copies already made from it
  int32_t cached = 0;                     // live nodes
  int64_t cache_hit_blocks = 0;
  int64_t cache_evictions = 0;

  std::map<TokenKey, int64_t>& children_of(int64_t parent) {
    return parent < 0 ? root : nodes[parent].children;
  }
  // Counts nodes whose whole subtree only the tree references (what eviction could free)
  // into *total, stopping as soon as it reaches `enough`; true when it did.
  bool evictable_at_least(const std::map<TokenKey, int64_t>& ch, int64_t enough, int64_t* total,
                          bool* all_free) const {
    *all_free = true;
    for (const auto& kv : ch) {
      const CacheNode& nd = nodes[kv.second];
      bool sub_free = false;
      if (evictable_at_least(nd.children, enough, total, &sub_free)) return true;
      if (sub_free && ref[nd.block] == 1) {
        if (++*total >= enough) return true;
      } else {
        *all_free = false;
      }
    }
    return false;
  }
  bool evictable_at_least(int64_t enough) const {
    if (enough <= 0) return true;
    int64_t total = 0;
    bool f = false;
    return evictable_at_least(root, enough, &total, &f);
  }
  // Evict the least recently used leaf only the tree references (ties: oldest node).
  bool evictable_node(int64_t id) const {
    const CacheNode& nd = nodes[id];
    return nd.live && nd.children.empty() && ref[nd.block] == 1;
  }
  void offer(int64_t id) {  // id may have become evictable
    if (id >= 0 && evictable_node(id)) cand.emplace(nodes[id].last_use, id);
  }
  bool evict_one() {
    while (!cand.empty()) {
      const auto [lu, id] = cand.top();
      cand.pop();
      if (!evictable_node(id) || nodes[id].last_use != lu) continue;  // stale entry
      CacheNode& nd = nodes[id];
      children_of(nd.parent).erase(nd.key);
      nd.live = false;
      --cached;
      node_of_block[nd.block] = -1;
      release(nd.block);
      ++cache_evictions;
      offer(nd.parent);  // it may be a leaf now
      return true;
    }
    return false;
  }
  // Frees what the tree can to cover a shortfall of `need` blocks; false if it cannot (then
  // nothing was evicted).
  bool make_room(int64_t need) {
    const int64_t short_by = need - nfree;
    if (short_by <= 0) return true;
    if (!evictable_at_least(short_by)) return false;
    for (int64_t i = 0; i < short_by; ++i) evict_one();
    return true;
  }

  int32_t take() {  // caller guarantees nfree > 0
    int32_t b = ring[head];
    head = (head + 1 == num_blocks) ? 0 : head + 1;
    --nfree;
    ref[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) {
      int32_t tail = head + nfree;
      if (tail >= num_blocks) tail -= num_blocks;
      ring[tail] = b;
      ++nfree;
    } else if (ref[b] == 1 && !node_of_block.empty()) {
      offer(node_of_block[b]);  // now held by the tree alone?
    }
  }
  // n % B, by a mask when B is a power of two (the usual 16, 32, 64).
  int32_t offset_of(int32_t n) const { return (B & (B - 1)) == 0 ? (n & (B - 1)) : n % B; }
  // New blocks a sequence of n tokens needs to grow by k tokens (block boundaries crossed).
  bool is_swapped(int64_t id) const { return swapped.count(id) != 0; }
  int64_t boundary_blocks(int32_t n, int32_t k) const {
    if (k <= 0) return 0;
    // positions n .. n+k-1 that are multiples of B
    int64_t first = (static_cast<int64_t>(n) + B - 1) / B;             // multiples >= n
    int64_t last = (static_cast<int64_t>(n) + k - 1) / B;              // multiples <= n+k-1
    return last - first + 1;
  }
};

using pa::fail;
using pa::ok;

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* init_free_order,
                       pa_bm** out) {
  if (!out) return fail(PA_ERR_INVALID_ARG, "pa_bm_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_create: num_blocks (%d) and block_size (%d) must be > 0",
                num_blocks, block_size);
  pa_bm* bm = new (std::nothrow) pa_bm();
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_create: out of host memory");
  try {
    bm->num_blocks = num_blocks;
    bm->B = block_size;
    bm->ref.assign(num_blocks, 0);
    bm->node_of_block.assign(num_blocks, -1);
    bm->ring.resize(num_blocks);
    if (init_free_order) {
      std::vector<char> seen(num_blocks, 0);
      for (int32_t i = 0; i < num_blocks; ++i) {
        int32_t b = init_free_order[i];
        if (b < 0 || b >= num_blocks || seen[b]) {
          delete bm;
          return fail(PA_ERR_INVALID_ARG,
                      "pa_bm_create: init_free_order is not a permutation (entry %d = %d)", i, b);
        }
        seen[b] = 1;
        bm->ring[i] = b;
      }
    } else {
      for (int32_t i = 0; i < num_blocks; ++i) bm->ring[i] = i;
    }
    bm->head = 0;
    bm->nfree = num_blocks;
  } catch (...) {
    delete bm;
    return fail(PA_ERR_INVALID_ARG, "pa_bm_create: out of host memory");
  }
  *out = bm;
  return ok();
}

pa_status pa_bm_destroy(pa_bm* bm) {
  delete bm;
  return ok();
}

pa_status pa_bm_add_seq(pa_bm* bm, int64_t seq_id, int32_t n_tokens, int32_t* slots_out) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq: NULL handle");
  if (n_tokens < 0) return fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq: n_tokens %d < 0", n_tokens);
  if (bm->seqs.count(seq_id) || bm->is_swapped(seq_id))
    return fail(PA_ERR_SEQ_EXISTS, "pa_bm_add_seq: sequence %lld exists", (long long)seq_id);
  const int64_t need = bm->boundary_blocks(0, n_tokens);
  if (!bm->make_room(need))
    return fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_add_seq: needs %lld blocks, %d free",
                (long long)need, bm->nfree);
  try {
    Seq s;
    s.blocks.reserve(need);
    for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
    s.n = n_tokens;
    if (slots_out) {
      const int32_t B = bm->B;
      for (int32_t j = 0; j < n_tokens; ++j) slots_out[j] = s.blocks[j / B] * B + j % B;
    }
    bm->seqs.emplace(seq_id, std::move(s));
  } catch (...) {
    return fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq: out of host memory");
  }
  return ok();
}

}  // extern "C"

namespace {

// One append call: tokens_each tokens for each of n_seqs sequences, in batch order; slots,
// copy-on-write pairs and (lens_out != nullptr) the lengths after the call.  Resolves every id
// and counts blocks and copies in a dry run first, so a failing call changes nothing.
pa_status append_batch(pa_bm* bm, const char* who, const int64_t* seq_ids, int32_t n_seqs,
                       int32_t tokens_each, int32_t* slots_out, int32_t* lens_out,
                       int32_t* copy_pairs_out, int32_t pairs_cap, int32_t* n_copies_out) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "%s: NULL handle", who);
  if (n_seqs < 0 || tokens_each < 0 || pairs_cap < 0)
    return fail(PA_ERR_INVALID_ARG, "%s: negative count", who);
  if (n_seqs > 0 && !seq_ids) return fail(PA_ERR_INVALID_ARG, "%s: seq_ids NULL", who);
  if (n_seqs > 0 && tokens_each > 0 && !slots_out)
    return fail(PA_ERR_INVALID_ARG, "%s: slots_out NULL", who);
  if (pairs_cap > 0 && !copy_pairs_out)
    return fail(PA_ERR_INVALID_ARG, "%s: copy_pairs_out NULL", who);
  if (n_copies_out) *n_copies_out = 0;
  const int32_t B = bm->B;

  // Dry run: resolve ids (or reuse the last call's resolution of the same ids), reject repeats
  // (a sequence named twice carries this call's stamp), count new blocks and copies in batch
  // order.  Only a shared last block can be copied, so only shared blocks are tracked.
  int64_t need = 0, copies = 0;
  try {
    const bool same = bm->batch_valid && bm->batch_erasures == bm->seq_erasures &&
                      bm->batch_ids.size() == static_cast<size_t>(n_seqs) &&
                      (n_seqs == 0 || std::memcmp(bm->batch_ids.data(), seq_ids,
                                                  sizeof(int64_t) * n_seqs) == 0);
    if (!same) {
      bm->batch_valid = false;
      bm->batch.resize(static_cast<size_t>(n_seqs));
      const uint64_t stamp = ++bm->epoch;
      for (int32_t i = 0; i < n_seqs; ++i) {
        auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end())
          return bm->is_swapped(seq_ids[i])
                     ? fail(PA_ERR_SWAPPED, "%s: sequence %lld is swapped out", who,
                            (long long)seq_ids[i])
                     : fail(PA_ERR_UNKNOWN_SEQ, "%s: unknown sequence %lld", who,
                            (long long)seq_ids[i]);
        Seq* s = &it->second;
        if (s->stamp == stamp)
          return fail(PA_ERR_INVALID_ARG, "%s: sequence %lld repeats in the batch", who,
                      (long long)seq_ids[i]);
        s->stamp = stamp;
        bm->batch[i] = s;
      }
      bm->batch_ids.assign(seq_ids, seq_ids + n_seqs);
      bm->batch_erasures = bm->seq_erasures;
      bm->batch_valid = true;
    }
    bm->cow.assign(static_cast<size_t>(n_seqs), 0);
    bm->dec.clear();
    for (int32_t i = 0; i < n_seqs && tokens_each > 0; ++i) {
      Seq* s = bm->batch[i];
      const int32_t off = bm->offset_of(s->n);
      if (off != 0) {
        const int32_t last = s->blocks.back();
        if (bm->ref[last] > 1) {
          int32_t& d = bm->dec[last];
          if (bm->ref[last] - d > 1) {
            bm->cow[i] = 1;
            ++d;
            ++copies;
            ++need;
          }
        }
      }
      if (static_cast<int64_t>(s->n) + tokens_each > INT32_MAX)
        return fail(PA_ERR_INVALID_ARG, "%s: sequence length overflows int32", who);
      const int64_t grow = tokens_each == 1 ? (off == 0) : bm->boundary_blocks(s->n, tokens_each);
      need += grow;
      // Capacity now (growing geometrically), so the commit below cannot throw half-way.
      const size_t want = s->blocks.size() + static_cast<size_t>(grow);
      if (s->blocks.capacity() < want) s->blocks.reserve(std::max(want, 2 * s->blocks.capacity()));
    }
  } catch (...) {
    bm->batch_valid = false;
    return fail(PA_ERR_INVALID_ARG, "%s: out of host memory", who);
  }
  if (copies > pairs_cap)
    return fail(PA_ERR_INVALID_ARG, "%s: %lld copy pairs needed, capacity %d", who,
                (long long)copies, pairs_cap);
  if (!bm->make_room(need))
    return fail(PA_ERR_OUT_OF_BLOCKS, "%s: needs %lld blocks, %d free", who, (long long)need,
                bm->nfree);

  // Commit.  The dry run reserved every table it grows; only the eviction heap (a block of
  // the prefix cache left referenced by the tree alone) can still allocate.
  int32_t np = 0;
  int64_t o = 0;
  try {
    for (int32_t i = 0; i < n_seqs; ++i) {
      Seq* s = bm->batch[i];
      if (tokens_each > 0) {
        if (bm->cow[i]) {
          const int32_t last = s->blocks.back();
          const int32_t fresh = bm->take();
          --bm->ref[last];  // stays >= 1: the dry run saw a count above one
          if (bm->ref[last] == 1) bm->offer(bm->node_of_block[last]);
          s->blocks.back() = fresh;
          copy_pairs_out[2 * np] = last;
          copy_pairs_out[2 * np + 1] = fresh;
          ++np;
          ++bm->cow_copies;
        }
        // position n sits in the last block at offset n % B (a new block when that is 0)
        int32_t off = bm->offset_of(s->n);
        for (int32_t t = 0; t < tokens_each; ++t) {
          if (off == 0) s->blocks.push_back(bm->take());
          slots_out[o++] = s->blocks.back() * B + off;
          off = off + 1 == B ? 0 : off + 1;
        }
        s->n += tokens_each;
      }
      if (lens_out) lens_out[i] = s->n;
    }
  } catch (...) {
    return fail(PA_ERR_INVALID_ARG, "%s: out of host memory during commit", who);
  }
  if (n_copies_out) *n_copies_out = np;
  return ok();
}

}  // namespace

extern "C" {

pa_status pa_bm_append_slots(pa_bm* bm, const int64_t* seq_ids, int32_t n_seqs,
                             int32_t tokens_each, int32_t* slots_out, int32_t* copy_pairs_out,
                             int32_t pairs_cap, int32_t* n_copies_out) {
  return append_batch(bm, "pa_bm_append_slots", seq_ids, n_seqs, tokens_each, slots_out, nullptr,
                      copy_pairs_out, pairs_cap, n_copies_out);
}

pa_status pa_bm_append_step(pa_bm* bm, const int64_t* seq_ids, int32_t n_seqs,
                            int32_t tokens_each, int32_t* slots_out, int32_t* lens_out,
                            int32_t* copy_pairs_out, int32_t pairs_cap, int32_t* n_copies_out) {
  if (n_seqs > 0 && !lens_out) return fail(PA_ERR_INVALID_ARG, "pa_bm_append_step: lens_out NULL");
  return append_batch(bm, "pa_bm_append_step", seq_ids, n_seqs, tokens_each, slots_out, lens_out,
                      copy_pairs_out, pairs_cap, n_copies_out);
}

pa_status pa_bm_fork(pa_bm* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_fork: NULL handle");
  auto it = bm->seqs.find(parent_id);
  if (it == bm->seqs.end())
    return bm->is_swapped(parent_id)
               ? fail(PA_ERR_SWAPPED, "pa_bm_fork: parent %lld is swapped out", (long long)parent_id)
               : fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_fork: unknown parent %lld", (long long)parent_id);
  if (bm->seqs.count(child_id) || bm->is_swapped(child_id))
    return fail(PA_ERR_SEQ_EXISTS, "pa_bm_fork: child %lld exists", (long long)child_id);
  try {
    Seq child = it->second;  // copy of table and length
    for (int32_t b : child.blocks) ++bm->ref[b];
    bm->seqs.emplace(child_id, std::move(child));
  } catch (...) {
    return fail(PA_ERR_INVALID_ARG, "pa_bm_fork: out of host memory");
  }
  ++bm->forks;
  return ok();
}

pa_status pa_bm_free_seq(pa_bm* bm, int64_t seq_id) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_free_seq: NULL handle");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) {
    if (bm->swapped.erase(seq_id)) return ok();  // a swapped sequence holds no blocks
    return fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_free_seq: unknown sequence %lld", (long long)seq_id);
  }
  for (int32_t b : it->second.blocks) bm->release(b);
  bm->seqs.erase(it);
  ++bm->seq_erasures;
  return ok();
}

pa_status pa_bm_block_tables(pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                             int32_t* tables_out, int32_t* ctx_lens_out) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_block_tables: NULL handle");
  if (n < 0 || max_blocks < 0) return fail(PA_ERR_INVALID_ARG, "pa_bm_block_tables: negative size");
  if (n > 0 && (!seq_ids || (max_blocks > 0 && !tables_out)))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_block_tables: NULL array");
  std::vector<const Seq*> rows(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end())
      return bm->is_swapped(seq_ids[i])
                 ? fail(PA_ERR_SWAPPED, "pa_bm_block_tables: sequence %lld is swapped out",
                        (long long)seq_ids[i])
                 : fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_block_tables: unknown sequence %lld",
                        (long long)seq_ids[i]);
    if (static_cast<int64_t>(it->second.blocks.size()) > max_blocks)
      return fail(PA_ERR_INVALID_ARG, "pa_bm_block_tables: sequence %lld holds %zu blocks > %d",
                  (long long)seq_ids[i], it->second.blocks.size(), max_blocks);
    rows[i] = &it->second;
  }
  for (int32_t i = 0; i < n; ++i) {
    int32_t* row = tables_out + static_cast<size_t>(i) * max_blocks;
    const size_t k = rows[i]->blocks.size();
    if (k) std::memcpy(row, rows[i]->blocks.data(), k * sizeof(int32_t));
    std::fill(row + k, row + max_blocks, -1);
    if (ctx_lens_out) ctx_lens_out[i] = rows[i]->n;
  }
  return ok();
}

pa_status pa_bm_seq_len(pa_bm* bm, int64_t seq_id, int32_t* n_out) {
  if (!bm || !n_out) return fail(PA_ERR_INVALID_ARG, "pa_bm_seq_len: NULL argument");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) {
    auto sw = bm->swapped.find(seq_id);
    if (sw == bm->swapped.end())
      return fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_seq_len: unknown sequence %lld", (long long)seq_id);
    *n_out = sw->second;
    return ok();
  }
  *n_out = it->second.n;
  return ok();
}

pa_status pa_bm_seq_lens(pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* lens_out) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_seq_lens: NULL handle");
  if (n < 0) return fail(PA_ERR_INVALID_ARG, "pa_bm_seq_lens: negative count");
  if (n > 0 && (!seq_ids || !lens_out)) return fail(PA_ERR_INVALID_ARG, "pa_bm_seq_lens: NULL array");
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) {
      auto sw = bm->swapped.find(seq_ids[i]);
      if (sw == bm->swapped.end())
        return fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_seq_lens: unknown sequence %lld",
                    (long long)seq_ids[i]);
      lens_out[i] = sw->second;
      continue;
    }
    lens_out[i] = it->second.n;
  }
  return ok();
}

pa_status pa_bm_share_groups(pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t max_members,
                             int32_t min_tokens, int32_t* groups_out, int32_t cap,
                             int32_t* n_groups_out) {
  if (!bm || !n_groups_out) return fail(PA_ERR_INVALID_ARG, "pa_bm_share_groups: NULL argument");
  *n_groups_out = 0;
  if (n < 0 || cap < 0 || max_members < 2 || max_members > 4 || min_tokens < 1)
    return fail(PA_ERR_INVALID_ARG,
                "pa_bm_share_groups: n %d, cap %d, max_members %d (2..4), min_tokens %d (>= 1)", n,
                cap, max_members, min_tokens);
  if (n > 0 && !seq_ids) return fail(PA_ERR_INVALID_ARG, "pa_bm_share_groups: seq_ids NULL");
  if (cap > 0 && !groups_out) return fail(PA_ERR_INVALID_ARG, "pa_bm_share_groups: groups_out NULL");
  try {
    std::vector<const Seq*> seq(static_cast<size_t>(n));
    for (int32_t i = 0; i < n; ++i) {
      auto it = bm->seqs.find(seq_ids[i]);
      if (it == bm->seqs.end())
        return bm->is_swapped(seq_ids[i])
                   ? fail(PA_ERR_SWAPPED, "pa_bm_share_groups: sequence %lld is swapped out",
                          (long long)seq_ids[i])
                   : fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_share_groups: unknown sequence %lld",
                          (long long)seq_ids[i]);
      seq[i] = &it->second;
    }
    // Tables in lexicographic order of their physical blocks: sequences with the longest
    // common physical prefix end up next to each other.
    std::vector<int32_t> ord(static_cast<size_t>(n));
    for (int32_t i = 0; i < n; ++i) ord[i] = i;
    std::sort(ord.begin(), ord.end(), [&](int32_t x, int32_t y) {
      return std::lexicographical_compare(seq[x]->blocks.begin(), seq[x]->blocks.end(),
                                          seq[y]->blocks.begin(), seq[y]->blocks.end()) ||
             (seq[x]->blocks == seq[y]->blocks && x < y);
    });
    // Tokens two sequences hold in the same physical blocks (positions below both lengths).
    auto shared = [&](int32_t x, int32_t y) -> int64_t {
      const auto& a = seq[x]->blocks;
      const auto& b = seq[y]->blocks;
      size_t k = 0;
      while (k < a.size() && k < b.size() && a[k] == b[k]) ++k;
      return std::min<int64_t>({static_cast<int64_t>(k) * bm->B, seq[x]->n, seq[y]->n});
    };
    std::vector<int64_t> adj(n > 0 ? static_cast<size_t>(n - 1) : 0);
    for (int32_t i = 0; i + 1 < n; ++i) adj[i] = shared(ord[i], ord[i + 1]);
    // The sorted order is the leaf order of the tree of common prefixes: a range whose adjacent
    // shared counts are all >= m is a node whose sequences share m tokens.  Walk it bottom-up:
    // at each node (m = the range's smallest adjacent count) group the sequences its subtrees
    // left over, max_members at a time; a remainder of r >= 2 is grouped here too when that
    // saves at least what its members could save one level up ((r - 1) m >= r m_parent),
    // otherwise it is left to the parent.  A group of k saves (k - 1) L reads.
    std::vector<std::pair<int64_t, std::vector<int32_t>>> groups;
    std::function<std::vector<int32_t>(int32_t, int32_t, int64_t)> walk =
        [&](int32_t lo, int32_t hi, int64_t m_parent) -> std::vector<int32_t> {
      if (hi - lo == 1) return {ord[lo]};
      int64_t m = INT64_MAX;
      for (int32_t i = lo; i + 1 < hi; ++i) m = std::min(m, adj[i]);
      std::vector<int32_t> left;
      int32_t start = lo;
      for (int32_t i = lo; i + 1 < hi; ++i)
        if (adj[i] == m) {
          auto sub = walk(start, i + 1, m);
          left.insert(left.end(), sub.begin(), sub.end());
          start = i + 1;
        }
      auto sub = walk(start, hi, m);
      left.insert(left.end(), sub.begin(), sub.end());
      if (m < min_tokens) return left;
      size_t k = 0;
      for (; left.size() - k >= static_cast<size_t>(max_members); k += max_members)
        groups.emplace_back(m, std::vector<int32_t>(left.begin() + k, left.begin() + k + max_members));
      const int64_t r = static_cast<int64_t>(left.size() - k);
      if (r >= 2 && (r - 1) * m >= r * m_parent) {
        groups.emplace_back(m, std::vector<int32_t>(left.begin() + k, left.end()));
        k = left.size();
      }
      return std::vector<int32_t>(left.begin() + k, left.end());
    };
    if (n > 1) (void)walk(0, n, 0);
    for (auto& g : groups) std::sort(g.second.begin(), g.second.end());
    std::sort(groups.begin(), groups.end(),
              [](const auto& x, const auto& y) { return x.second[0] < y.second[0]; });
    *n_groups_out = static_cast<int32_t>(groups.size());
    if (static_cast<int32_t>(groups.size()) > cap)
      return fail(PA_ERR_INVALID_ARG, "pa_bm_share_groups: %zu groups, capacity %d",
                  groups.size(), cap);
    for (size_t g = 0; g < groups.size(); ++g) {
      int32_t* row = groups_out + g * 5;
      row[0] = static_cast<int32_t>(std::min<int64_t>(groups[g].first, INT32_MAX));
      for (int k = 0; k < 4; ++k)
        row[1 + k] = k < static_cast<int>(groups[g].second.size()) ? groups[g].second[k] : -1;
    }
  } catch (...) {
    return fail(PA_ERR_INVALID_ARG, "pa_bm_share_groups: out of host memory");
  }
  return ok();
}

pa_status pa_bm_refcount(pa_bm* bm, int32_t block, int32_t* out) {
  if (!bm || !out) return fail(PA_ERR_INVALID_ARG, "pa_bm_refcount: NULL argument");
  if (block < 0 || block >= bm->num_blocks)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_refcount: block %d outside [0, %d)", block,
                bm->num_blocks);
  *out = bm->ref[block];
  return ok();
}

pa_status pa_bm_free_list(pa_bm* bm, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!bm || !n_out) return fail(PA_ERR_INVALID_ARG, "pa_bm_free_list: NULL argument");
  if (cap < 0 || (cap > 0 && !out)) return fail(PA_ERR_INVALID_ARG, "pa_bm_free_list: bad capacity");
  const int32_t k = std::min(cap, bm->nfree);
  for (int32_t i = 0; i < k; ++i) {
    int32_t idx = bm->head + i;
    if (idx >= bm->num_blocks) idx -= bm->num_blocks;
    out[i] = bm->ring[idx];
  }
  *n_out = bm->nfree;
  return ok();
}

pa_status pa_bm_stats(pa_bm* bm, pa_bm_stats_t* out) {
  if (!bm || !out) return fail(PA_ERR_INVALID_ARG, "pa_bm_stats: NULL argument");
  pa_bm_stats_t st{};
  st.num_blocks = bm->num_blocks;
  st.block_size = bm->B;
  st.free_blocks = bm->nfree;
  for (int32_t r : bm->ref) {
    if (r >= 1) ++st.used_blocks;
    if (r >= 2) ++st.shared_blocks;
  }
  st.num_seqs = static_cast<int32_t>(bm->seqs.size());
  for (const auto& kv : bm->seqs) {
    st.logical_blocks += static_cast<int64_t>(kv.second.blocks.size());
    st.live_tokens += kv.second.n;
  }
  st.tail_waste_slots = st.logical_blocks * bm->B - st.live_tokens;
  st.forks = bm->forks;
  st.cow_copies = bm->cow_copies;
  st.usage = static_cast<double>(st.used_blocks) / bm->num_blocks;
  st.swapped_seqs = static_cast<int32_t>(bm->swapped.size());
  for (const auto& kv : bm->swapped) st.swapped_tokens += kv.second;
  st.swap_outs = bm->swap_outs;
  st.swap_ins = bm->swap_ins;
  st.cached_blocks = bm->cached;
  st.cache_hit_blocks = bm->cache_hit_blocks;
  st.cache_evictions = bm->cache_evictions;
  *out = st;
  return ok();
}

pa_status pa_bm_swap_out(pa_bm* bm, int64_t seq_id, int32_t* blocks_out, int32_t cap,
                         int32_t* n_out) {
  if (!bm || !n_out) return fail(PA_ERR_INVALID_ARG, "pa_bm_swap_out: NULL argument");
  *n_out = 0;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end())
    return bm->is_swapped(seq_id)
               ? fail(PA_ERR_SWAPPED, "pa_bm_swap_out: sequence %lld is already swapped out",
                      (long long)seq_id)
               : fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_swap_out: unknown sequence %lld", (long long)seq_id);
  const auto& blocks = it->second.blocks;
  const int32_t k = static_cast<int32_t>(blocks.size());
  *n_out = k;
  if (cap < k || (k > 0 && !blocks_out))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_swap_out: %d blocks, capacity %d", k, cap);
  try {
    bm->swapped.reserve(bm->swapped.size() + 1);
    bm->swapped.emplace(seq_id, it->second.n);
  } catch (...) {
    return fail(PA_ERR_INVALID_ARG, "pa_bm_swap_out: out of host memory");
  }
  for (int32_t i = 0; i < k; ++i) blocks_out[i] = blocks[i];
  for (int32_t b : blocks) bm->release(b);
  bm->seqs.erase(it);
  ++bm->seq_erasures;
  ++bm->swap_outs;
  return ok();
}

pa_status pa_bm_swap_in(pa_bm* bm, int64_t seq_id, int32_t* blocks_out, int32_t cap,
                        int32_t* n_out) {
  if (!bm || !n_out) return fail(PA_ERR_INVALID_ARG, "pa_bm_swap_in: NULL argument");
  *n_out = 0;
  auto sw = bm->swapped.find(seq_id);
  if (sw == bm->swapped.end())
    return bm->seqs.count(seq_id)
               ? fail(PA_ERR_INVALID_ARG, "pa_bm_swap_in: sequence %lld is not swapped out",
                      (long long)seq_id)
               : fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_swap_in: unknown sequence %lld", (long long)seq_id);
  const int32_t n = sw->second;
  const int32_t k = static_cast<int32_t>(bm->boundary_blocks(0, n));
  *n_out = k;
  if (cap < k || (k > 0 && !blocks_out))
    return fail(PA_ERR_INVALID_ARG, "pa_bm_swap_in: %d blocks, capacity %d", k, cap);
  if (!bm->make_room(k))
    return fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_swap_in: needs %d blocks, %d free", k, bm->nfree);
  try {
    Seq s;
    s.blocks.reserve(k);
    bm->seqs.reserve(bm->seqs.size() + 1);
    for (int32_t i = 0; i < k; ++i) s.blocks.push_back(bm->take());
    s.n = n;
    for (int32_t i = 0; i < k; ++i) blocks_out[i] = s.blocks[i];
    bm->seqs.emplace(seq_id, std::move(s));
  } catch (...) {
    // Unreachable in practice (the capacities are reserved first).
    return fail(PA_ERR_INVALID_ARG, "pa_bm_swap_in: out of host memory");
  }
  bm->swapped.erase(sw);
  ++bm->swap_ins;
  return ok();
}

pa_status pa_bm_truncate(pa_bm* bm, int64_t seq_id, int32_t n_keep) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_truncate: NULL handle");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end())
    return bm->is_swapped(seq_id)
               ? fail(PA_ERR_SWAPPED, "pa_bm_truncate: sequence %lld is swapped out", (long long)seq_id)
               : fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_truncate: unknown sequence %lld", (long long)seq_id);
  Seq& s = it->second;
  if (n_keep < 0 || n_keep > s.n)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_truncate: n_keep %d outside [0, %d]", n_keep, s.n);
  const size_t keep = static_cast<size_t>(bm->boundary_blocks(0, n_keep));
  for (size_t i = keep; i < s.blocks.size(); ++i) bm->release(s.blocks[i]);
  s.blocks.resize(keep);
  s.n = n_keep;
  return ok();
}

pa_status pa_bm_add_seq_cached(pa_bm* bm, int64_t seq_id, const int32_t* tokens,
                               int32_t n_tokens, int32_t* slots_out, int32_t* n_cached_out) {
  if (!bm || !n_cached_out) return fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq_cached: NULL argument");
  *n_cached_out = 0;
  if (n_tokens < 0) return fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq_cached: n_tokens %d < 0", n_tokens);
  if (n_tokens > 0 && !tokens) return fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq_cached: tokens NULL");
  if (bm->seqs.count(seq_id) || bm->is_swapped(seq_id))
    return fail(PA_ERR_SEQ_EXISTS, "pa_bm_add_seq_cached: sequence %lld exists", (long long)seq_id);
  const int32_t B = bm->B;
  std::vector<int64_t> matched;
  try {
    const std::map<TokenKey, int64_t>* ch = &bm->root;
    TokenKey key(B);
    for (int32_t j = 0; j + 1 <= n_tokens / B; ++j) {
      std::copy(tokens + static_cast<size_t>(j) * B, tokens + static_cast<size_t>(j + 1) * B,
                key.begin());
      auto it = ch->find(key);
      if (it == ch->end()) break;
      matched.push_back(it->second);
      ch = &bm->nodes[it->second].children;
    }
  } catch (...) {
    return fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq_cached: out of host memory");
  }
  const int64_t m = static_cast<int64_t>(matched.size());
  const int64_t need = bm->boundary_blocks(0, n_tokens) - m;
  // The matched blocks are referenced before anything is evicted, so they cannot be.
  for (int64_t id : matched) ++bm->ref[bm->nodes[id].block];
  auto undo = [&] {
    for (int64_t id : matched) {
      --bm->ref[bm->nodes[id].block];
      bm->offer(id);
    }
  };
  if (need > bm->nfree && !bm->evictable_at_least(need - bm->nfree)) {
    undo();
    return fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_add_seq_cached: needs %lld blocks, %d free",
                (long long)need, bm->nfree);
  }
  try {
    Seq s;
    s.blocks.reserve(static_cast<size_t>(m + need));
    bm->seqs.reserve(bm->seqs.size() + 1);
    for (int64_t id : matched) {
      s.blocks.push_back(bm->nodes[id].block);
      bm->nodes[id].last_use = bm->tick;
    }
    ++bm->tick;
    bm->make_room(need);  // cannot fail: checked above
    for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
    s.n = n_tokens;
    if (slots_out)
      for (int32_t j = 0; j < n_tokens; ++j) slots_out[j] = s.blocks[j / B] * B + j % B;
    bm->seqs.emplace(seq_id, std::move(s));
  } catch (...) {
    undo();
    return fail(PA_ERR_INVALID_ARG, "pa_bm_add_seq_cached: out of host memory");
  }
  bm->cache_hit_blocks += m;
  *n_cached_out = static_cast<int32_t>(m * B);
  return ok();
}

pa_status pa_bm_cache_insert(pa_bm* bm, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                             int32_t* n_added_out) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "pa_bm_cache_insert: NULL handle");
  if (n_added_out) *n_added_out = 0;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end())
    return bm->is_swapped(seq_id)
               ? fail(PA_ERR_SWAPPED, "pa_bm_cache_insert: sequence %lld is swapped out", (long long)seq_id)
               : fail(PA_ERR_UNKNOWN_SEQ, "pa_bm_cache_insert: unknown sequence %lld", (long long)seq_id);
  const Seq& sq = it->second;
  if (n_tokens < 0 || n_tokens > sq.n)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_cache_insert: n_tokens %d outside [0, %d]", n_tokens, sq.n);
  if (n_tokens > 0 && !tokens) return fail(PA_ERR_INVALID_ARG, "pa_bm_cache_insert: tokens NULL");
  const int32_t B = bm->B;
  const int32_t k = n_tokens / B;
  int32_t added = 0;
  try {
    int64_t parent = -1;
    TokenKey key(B);
    for (int32_t j = 0; j < k; ++j) {
      std::copy(tokens + static_cast<size_t>(j) * B, tokens + static_cast<size_t>(j + 1) * B,
                key.begin());
      auto& ch = bm->children_of(parent);
      auto f = ch.find(key);
      int64_t id;
      if (f == ch.end()) {
        id = static_cast<int64_t>(bm->nodes.size());
        CacheNode nd;
        nd.block = sq.blocks[j];
        nd.key = key;
        nd.parent = parent;
        bm->nodes.push_back(std::move(nd));
        bm->children_of(parent).emplace(key, id);
        ++bm->ref[sq.blocks[j]];
        bm->node_of_block[sq.blocks[j]] = id;
        ++bm->cached;
        ++added;
      } else {
        id = f->second;
      }
      bm->nodes[id].last_use = bm->tick;
      bm->offer(id);  // a touched node keeps its place only with its new use
      parent = id;
    }
  } catch (...) {
    // A partial insert leaves a consistent tree (every added node holds its reference).
    return fail(PA_ERR_INVALID_ARG, "pa_bm_cache_insert: out of host memory");
  }
  ++bm->tick;
  if (n_added_out) *n_added_out = added;
  return ok();
}

pa_status pa_bm_cache_evict(pa_bm* bm, int32_t n_blocks, int32_t* n_evicted_out) {
  if (!bm || !n_evicted_out) return fail(PA_ERR_INVALID_ARG, "pa_bm_cache_evict: NULL argument");
  if (n_blocks < 0) return fail(PA_ERR_INVALID_ARG, "pa_bm_cache_evict: n_blocks %d < 0", n_blocks);
  int32_t done = 0;
  while (done < n_blocks && bm->evict_one()) ++done;
  *n_evicted_out = done;
  return ok();
}

pa_status pa_bm_accounting(const int32_t* lens, int32_t n, int32_t block_size,
                           int32_t max_seq_len, pa_accounting_t* out) {
  if (!out || (n > 0 && !lens)) return fail(PA_ERR_INVALID_ARG, "pa_bm_accounting: NULL argument");
  if (n <= 0 || block_size <= 0 || max_seq_len <= 0)
    return fail(PA_ERR_INVALID_ARG, "pa_bm_accounting: n, block_size and max_seq_len must be > 0");
  int64_t actual = 0, blocks = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (lens[i] < 0) return fail(PA_ERR_INVALID_ARG, "pa_bm_accounting: length %d < 0", lens[i]);
    actual += lens[i];
    blocks += (static_cast<int64_t>(lens[i]) + block_size - 1) / block_size;
  }
  pa_accounting_t r{};
  r.total_actual_tokens = actual;
  r.paged_slots = blocks * block_size;
  r.naive_slots = static_cast<int64_t>(max_seq_len) * n;
  if (r.paged_slots == 0) return fail(PA_ERR_INVALID_ARG, "pa_bm_accounting: all lengths are zero");
  r.paged_fragmentation_pct =
      100.0 * static_cast<double>(r.paged_slots - actual) / static_cast<double>(r.paged_slots);
  r.naive_fragmentation_pct =
      100.0 * static_cast<double>(r.naive_slots - actual) / static_cast<double>(r.naive_slots);
  r.memory_reduction_factor = static_cast<double>(r.naive_slots) / static_cast<double>(r.paged_slots);
  *out = r;
  return ok();
}

pa_status pa_validate_tables(const int32_t* tables, const int32_t* ctx_lens, int32_t S,
                             int32_t max_blocks, int32_t block_size, int32_t num_blocks) {
  if (S < 0 || max_blocks <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "pa_validate_tables: bad sizes");
  if (S > 0 && (!tables || !ctx_lens)) return fail(PA_ERR_INVALID_ARG, "pa_validate_tables: NULL");
  for (int32_t s = 0; s < S; ++s) {
    const int64_t n = ctx_lens[s];
    if (n < 1 || n > static_cast<int64_t>(max_blocks) * block_size)
      return fail(PA_ERR_INVALID_ARG, "pa_validate_tables: row %d: ctx_len %lld outside [1, %lld]",
                  s, (long long)n, (long long)max_blocks * block_size);
    const int64_t used = (n + block_size - 1) / block_size;
    const int32_t* row = tables + static_cast<size_t>(s) * max_blocks;
    for (int64_t j = 0; j < used; ++j)
      if (row[j] < 0 || row[j] >= num_blocks)
        return fail(PA_ERR_INVALID_ARG, "pa_validate_tables: row %d entry %lld = %d outside [0, %d)",
                    s, (long long)j, row[j], num_blocks);
  }
  return ok();
}

}  // extern "C"
