// host_runtime.cpp - host side of libpagedkv: status names, version, table
// validation and the block manager (free list, reference counts, per-sequence
// tables with fork, copy-on-write, swapping and automatic prefix caching).
// CPU only; no device calls.
//
// Sources cited by tag and section:
//   [pofe]   "PagedAttention: paging the KV cache"
//   [lesson] "PagedAttention" lesson in "How Text Is Generated"
//   [note]   "PagedAttention: Manage the Cache Without Moving the Sequence"
//   [claims] "Paged Attention" claims page
//   [arch]   "PagedAttention: Virtual-Memory KV Cache Management, Continuous
//            Batching, and PyTorch Architecture"
#include <stdint.h>

#include <algorithm>
#include <iterator>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"

extern "C" const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_NO_FREE_BLOCK: return "PKV_ERR_NO_FREE_BLOCK";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    case PKV_ERR_ORDER: return "PKV_ERR_ORDER";
    default: return "PKV_ERR_UNKNOWN";
  }
}

extern "C" int pkv_version(void) { return 100; }  // 0.1.0

extern "C" int pkv_validate_tables(const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* context_lens, int num_seqs, int num_blocks,
                                   int block_size, int* bad_seq_out) {
  if (bad_seq_out) *bad_seq_out = -1;
  if (num_seqs < 0 || max_blocks_per_seq < 1 || num_blocks < 1 || block_size < 1)
    return PKV_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!block_tables || !context_lens)) return PKV_ERR_INVALID_ARG;
  for (int s = 0; s < num_seqs; ++s) {
    const long long len = context_lens[s];
    const long long nb = len <= 0 ? 0 : (len + block_size - 1) / block_size;
    bool ok = nb <= max_blocks_per_seq;
    for (long long j = 0; ok && j < nb; ++j) {
      const int id = block_tables[(size_t)s * max_blocks_per_seq + j];
      ok = id >= 0 && id < num_blocks;
    }
    if (!ok) {
      if (bad_seq_out) *bad_seq_out = s;
      return PKV_ERR_INVALID_ARG;
    }
  }
  return PKV_OK;
}

// ---------------------------------------------------------------------------
// Block manager.  Semantics of [pofe] "Minimal implementation" (BlockPool and
// Sequence) and the decode-step pseudocode of [pofe] "How it works".
// ---------------------------------------------------------------------------
struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> table;
    int len = 0;
    bool live = false;
    bool swapped = false;   // preempted by swapping: no blocks, length kept
  };
  int num_blocks = 0;
  int block_size = 0;
  std::vector<int32_t> free_list;   // LIFO: ids handed out from the back
  std::vector<int32_t> ref;
  std::vector<Seq> seqs;

  // Automatic prefix caching ([lesson] "Sharing, and the reference counting
  // it needs": block-aligned prefixes of token ids in a global table; [claims]
  // "Paged Attention": a hit needs an unbroken matching prefix).  A full
  // prompt block is keyed by a 64-bit chain over the prefix: key_j =
  // mix(key_{j-1}, tokens of block j).  An entry keeps its parent key and its
  // own token ids, and a lookup checks both, so a false hit needs two whole
  // prefixes whose 64-bit chains collide.  A cached block whose count falls
  // to 0 keeps its entry and waits in `lru` (oldest first) until a hit
  // revives it or an allocation with an empty free list evicts it.
  struct CacheEntry {
    int32_t block;
    uint64_t parent;
    std::vector<int32_t> tokens;
  };
  std::unordered_map<uint64_t, CacheEntry> cache;
  std::vector<uint64_t> key_of;   // per block: its key, when cached[b]
  std::vector<char> cached;
  std::list<int32_t> lru;
  std::vector<std::list<int32_t>::iterator> lru_pos;

  // SplitMix64 finaliser (Steele, Lea and Flood, 2014) as the mixing step.
  static uint64_t mix(uint64_t x) {
    x += 0x9e3779b97f4a7c15ULL;
    x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ULL;
    x = (x ^ (x >> 27)) * 0x94d049bb133111ebULL;
    return x ^ (x >> 31);
  }
  static uint64_t chain(uint64_t parent, const int32_t* t, int n) {
    uint64_t k = mix(parent ^ 0x70726566697843ULL);
    for (int i = 0; i < n; ++i) k = mix(k ^ (uint64_t)(uint32_t)t[i]);
    return k;
  }
  // Blocks an allocation may take: free ones and evictable cached ones.
  long long allocatable() const { return (long long)free_list.size() + (long long)lru.size(); }

  bool block_ok(int b) const { return b >= 0 && b < num_blocks; }
  bool seq_ok(int s) const { return s >= 0 && s < (int)seqs.size() && seqs[s].live; }
  // A live sequence that holds its blocks (not swapped out).
  bool seq_resident(int s) const { return seq_ok(s) && !seqs[s].swapped; }

  int alloc() {   // caller has checked that allocatable() > 0
    int i;
    if (!free_list.empty()) {
      i = free_list.back();
      free_list.pop_back();
    } else {          // evict the oldest cached block with count 0
      i = lru.front();
      lru.pop_front();
      cache.erase(key_of[i]);
      cached[i] = 0;
    }
    ref[i] = 1;
    return i;
  }
  void release(int i) {
    if (--ref[i] == 0) {
      if (cached[i]) {
        lru.push_back(i);
        lru_pos[i] = std::prev(lru.end());
      } else {
        free_list.push_back(i);
      }
    }
  }

  // Blocks the next append of sequence s needs from the free list (0 or 1):
  // one at a block boundary, one for copy-on-write of a shared partial block.
  int append_need(const Seq& q) const {
    if (q.len % block_size == 0) return 1;
    return ref[q.table.back()] > 1 ? 1 : 0;
  }

  void append(Seq& q, int* block, int* slot, int* cow_src) {
    *cow_src = -1;
    if (q.len % block_size == 0) {
      q.table.push_back(alloc());
    } else if (ref[q.table.back()] > 1) {
      // [arch] "4. Automatic Prefix Caching (APC) and Copy-on-Write (CoW)":
      // fresh block, caller copies the B slots, old count - 1, remap.
      const int old = q.table.back();
      const int fresh = alloc();
      release(old);
      q.table.back() = fresh;
      *cow_src = old;
    }
    *block = q.table.back();
    *slot = q.len % block_size;
    q.len += 1;
  }
};

extern "C" int pkv_bm_create(int num_blocks, int block_size, pkv_block_manager** out) {
  if (!out) return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1) return PKV_ERR_INVALID_ARG;
  pkv_block_manager* bm = new (std::nothrow) pkv_block_manager();
  if (!bm) return PKV_ERR_INVALID_ARG;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->free_list.resize(num_blocks);
    for (int i = 0; i < num_blocks; ++i) bm->free_list[i] = i;
    bm->ref.assign(num_blocks, 0);
    bm->key_of.assign(num_blocks, 0);
    bm->cached.assign(num_blocks, 0);
    bm->lru_pos.resize(num_blocks);
  } catch (...) {
    delete bm;
    return PKV_ERR_INVALID_ARG;
  }
  *out = bm;
  return PKV_OK;
}

extern "C" void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

extern "C" int pkv_bm_num_free(const pkv_block_manager* bm) {
  if (!bm) return PKV_ERR_INVALID_ARG;
  return (int)bm->allocatable();
}

extern "C" int pkv_bm_refcount(const pkv_block_manager* bm, int block) {
  if (!bm || !bm->block_ok(block)) return PKV_ERR_INVALID_ARG;
  return bm->ref[block];
}

extern "C" int pkv_bm_alloc(pkv_block_manager* bm, int* block_out) {
  if (!bm || !block_out) return PKV_ERR_INVALID_ARG;
  if (bm->allocatable() == 0) return PKV_ERR_NO_FREE_BLOCK;
  *block_out = bm->alloc();
  return PKV_OK;
}

extern "C" int pkv_bm_share(pkv_block_manager* bm, int block) {
  if (!bm || !bm->block_ok(block) || bm->ref[block] <= 0) return PKV_ERR_INVALID_ARG;
  bm->ref[block] += 1;
  return PKV_OK;
}

extern "C" int pkv_bm_release(pkv_block_manager* bm, int block) {
  if (!bm || !bm->block_ok(block) || bm->ref[block] <= 0) return PKV_ERR_INVALID_ARG;
  bm->release(block);
  return PKV_OK;
}

extern "C" int pkv_bm_seq_new(pkv_block_manager* bm, int* seq_out) {
  if (!bm || !seq_out) return PKV_ERR_INVALID_ARG;
  try {
    bm->seqs.emplace_back();
  } catch (...) {
    return PKV_ERR_INVALID_ARG;
  }
  bm->seqs.back().live = true;
  *seq_out = (int)bm->seqs.size() - 1;
  return PKV_OK;
}

extern "C" int pkv_bm_seq_extend(pkv_block_manager* bm, int seq, int n_tokens) {
  if (!bm || !bm->seq_resident(seq) || n_tokens < 0) return PKV_ERR_INVALID_ARG;
  auto& q = bm->seqs[seq];
  const int b = bm->block_size;
  if (q.len % b != 0 && bm->ref[q.table.back()] > 1) return PKV_ERR_INVALID_ARG;
  const long long total = (long long)q.len + n_tokens;
  if (total > 0x7fffffffLL) return PKV_ERR_INVALID_ARG;
  const long long need = (total + b - 1) / b - (long long)q.table.size();
  if (need > bm->allocatable()) return PKV_ERR_NO_FREE_BLOCK;
  for (long long i = 0; i < need; ++i) q.table.push_back(bm->alloc());
  q.len = (int)total;
  return PKV_OK;
}

extern "C" int pkv_bm_seq_adopt_prefix(pkv_block_manager* bm, int seq, int src, int n_blocks) {
  if (!bm || !bm->seq_resident(seq) || !bm->seq_resident(src) || n_blocks < 0 || seq == src)
    return PKV_ERR_INVALID_ARG;
  auto& q = bm->seqs[seq];
  const auto& from = bm->seqs[src];
  if (!q.table.empty() || q.len != 0) return PKV_ERR_INVALID_ARG;
  if ((long long)n_blocks * bm->block_size > from.len) return PKV_ERR_INVALID_ARG;
  for (int j = 0; j < n_blocks; ++j) {
    bm->ref[from.table[j]] += 1;
    q.table.push_back(from.table[j]);
  }
  q.len = n_blocks * bm->block_size;
  return PKV_OK;
}

extern "C" int pkv_bm_seq_fork(pkv_block_manager* bm, int parent, int* child_out) {
  if (!bm || !bm->seq_resident(parent) || !child_out) return PKV_ERR_INVALID_ARG;
  int child = -1;
  int st = pkv_bm_seq_new(bm, &child);
  if (st != PKV_OK) return st;
  auto& c = bm->seqs[child];
  const auto& par = bm->seqs[parent];   // reference taken after the push_back
  c.table = par.table;
  c.len = par.len;
  for (int32_t b : c.table) bm->ref[b] += 1;
  *child_out = child;
  return PKV_OK;
}

extern "C" int pkv_bm_seq_append_slot(pkv_block_manager* bm, int seq, int* block_out,
                                      int* slot_out, int* cow_src_out) {
  if (!bm || !bm->seq_resident(seq) || !block_out || !slot_out || !cow_src_out)
    return PKV_ERR_INVALID_ARG;
  auto& q = bm->seqs[seq];
  if (q.len == 0x7fffffff) return PKV_ERR_INVALID_ARG;
  if (bm->append_need(q) > bm->allocatable()) return PKV_ERR_NO_FREE_BLOCK;
  bm->append(q, block_out, slot_out, cow_src_out);
  return PKV_OK;
}

extern "C" int pkv_bm_append_batch(pkv_block_manager* bm, const int* seqs, int n,
                                   int32_t* block_out, int32_t* slot_out, int32_t* cow_src_out,
                                   int32_t* cow_dst_out, int* num_cow_out) {
  if (!bm || n < 0 || !num_cow_out) return PKV_ERR_INVALID_ARG;
  *num_cow_out = 0;
  if (n == 0) return PKV_OK;
  if (!seqs || !block_out || !slot_out || !cow_src_out || !cow_dst_out) return PKV_ERR_INVALID_ARG;
  // All or nothing: a sequence may appear once, and the free list must cover
  // every allocation of the step before anything changes.
  long long need = 0;
  std::vector<char> seen;
  try {
    seen.assign(bm->seqs.size(), 0);
  } catch (...) {
    return PKV_ERR_INVALID_ARG;
  }
  for (int i = 0; i < n; ++i) {
    const int s = seqs[i];
    if (!bm->seq_resident(s) || seen[s] || bm->seqs[s].len == 0x7fffffff)
      return PKV_ERR_INVALID_ARG;
    seen[s] = 1;
    need += bm->append_need(bm->seqs[s]);
  }
  if (need > bm->allocatable()) return PKV_ERR_NO_FREE_BLOCK;
  int ncow = 0;
  for (int i = 0; i < n; ++i) {
    int blk, slot, cow;
    bm->append(bm->seqs[seqs[i]], &blk, &slot, &cow);
    block_out[i] = blk;
    slot_out[i] = slot;
    if (cow >= 0) {
      cow_src_out[ncow] = cow;
      cow_dst_out[ncow] = blk;
      ++ncow;
    }
  }
  *num_cow_out = ncow;
  return PKV_OK;
}

extern "C" int pkv_bm_seq_free(pkv_block_manager* bm, int seq) {
  if (!bm || !bm->seq_ok(seq)) return PKV_ERR_INVALID_ARG;
  auto& q = bm->seqs[seq];
  for (int32_t b : q.table) bm->release(b);
  q.table.clear();
  q.table.shrink_to_fit();
  q.len = 0;
  q.live = false;
  q.swapped = false;
  return PKV_OK;
}

// Preemption by swapping ([pofe] "When memory runs out": whole sequences, all
// or none of their blocks, are copied to CPU memory and back).  swap_out hands
// back the table (the blocks to copy out; host slot i = logical block i) and
// releases every block, shared ones included; swap_in allocates fresh blocks
// for the kept length, all or none.
extern "C" int pkv_bm_seq_swap_out(pkv_block_manager* bm, int seq, int32_t* blocks_out, int cap,
                                   int* n_out) {
  if (!bm || !bm->seq_resident(seq) || !n_out || cap < 0) return PKV_ERR_INVALID_ARG;
  auto& q = bm->seqs[seq];
  const int n = (int)q.table.size();
  if (n > cap || (n > 0 && !blocks_out)) return PKV_ERR_INVALID_ARG;
  for (int j = 0; j < n; ++j) blocks_out[j] = q.table[j];
  for (int32_t b : q.table) bm->release(b);
  q.table.clear();
  q.swapped = true;
  *n_out = n;
  return PKV_OK;
}

extern "C" int pkv_bm_seq_swap_in(pkv_block_manager* bm, int seq, int32_t* blocks_out, int cap,
                                  int* n_out) {
  if (!bm || !bm->seq_ok(seq) || !bm->seqs[seq].swapped || !n_out || cap < 0)
    return PKV_ERR_INVALID_ARG;
  auto& q = bm->seqs[seq];
  const int need = (int)(((long long)q.len + bm->block_size - 1) / bm->block_size);
  if (need > cap || (need > 0 && !blocks_out)) return PKV_ERR_INVALID_ARG;
  if (need > bm->allocatable()) return PKV_ERR_NO_FREE_BLOCK;
  try {
    q.table.reserve(need);
  } catch (...) {
    return PKV_ERR_INVALID_ARG;
  }
  for (int j = 0; j < need; ++j) {
    q.table.push_back(bm->alloc());
    blocks_out[j] = q.table.back();
  }
  q.swapped = false;
  *n_out = need;
  return PKV_OK;
}

extern "C" int pkv_bm_seq_is_swapped(const pkv_block_manager* bm, int seq) {
  if (!bm || !bm->seq_ok(seq)) return PKV_ERR_INVALID_ARG;
  return bm->seqs[seq].swapped ? 1 : 0;
}

extern "C" int pkv_bm_seq_len(const pkv_block_manager* bm, int seq) {
  if (!bm || !bm->seq_ok(seq)) return PKV_ERR_INVALID_ARG;
  return bm->seqs[seq].len;
}

extern "C" int pkv_bm_seq_num_blocks(const pkv_block_manager* bm, int seq) {
  if (!bm || !bm->seq_ok(seq)) return PKV_ERR_INVALID_ARG;
  return (int)bm->seqs[seq].table.size();
}

extern "C" int pkv_bm_seq_table(const pkv_block_manager* bm, int seq, int32_t* out, int cap) {
  if (!bm || !bm->seq_ok(seq) || cap < 0 || (cap > 0 && !out)) return PKV_ERR_INVALID_ARG;
  const auto& t = bm->seqs[seq].table;
  const int n = (int)t.size() < cap ? (int)t.size() : cap;
  for (int i = 0; i < n; ++i) out[i] = t[i];
  return n;
}

extern "C" int pkv_bm_export_tables(const pkv_block_manager* bm, const int* seqs, int n,
                                    int32_t* out, int ld, int32_t* lens_out) {
  if (!bm || n < 0 || ld < 1) return PKV_ERR_INVALID_ARG;
  if (n == 0) return PKV_OK;
  if (!seqs || !out || !lens_out) return PKV_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i) {
    if (!bm->seq_resident(seqs[i]) || (int)bm->seqs[seqs[i]].table.size() > ld)
      return PKV_ERR_INVALID_ARG;
  }
  for (int i = 0; i < n; ++i) {
    const auto& q = bm->seqs[seqs[i]];
    int32_t* row = out + (size_t)i * ld;
    const int nb = (int)q.table.size();
    for (int j = 0; j < nb; ++j) row[j] = q.table[j];
    for (int j = nb; j < ld; ++j) row[j] = -1;
    lens_out[i] = q.len;
  }
  return PKV_OK;
}

// Admission with prefix caching: share the cached blocks of the longest
// cached block-aligned prefix of `tokens`, allocate the rest (all or none),
// and enter the new full blocks under their prefixes (the caller writes
// their positions before any attention reads them).  A prefix already
// cached under another block, out of the walk's reach because its parent
// was evicted, keeps that block.
extern "C" int pkv_bm_seq_admit_prompt(pkv_block_manager* bm, int seq, const int32_t* tokens,
                                       int n_tokens, int* cached_tokens_out) {
  if (!bm || !bm->seq_resident(seq) || n_tokens < 0 || !cached_tokens_out ||
      (n_tokens > 0 && !tokens))
    return PKV_ERR_INVALID_ARG;
  auto& q = bm->seqs[seq];
  if (!q.table.empty() || q.len != 0) return PKV_ERR_INVALID_ARG;
  const int b = bm->block_size;
  const int full = n_tokens / b;
  std::vector<int32_t> hits;
  std::vector<uint64_t> keys;
  try {
    keys.reserve(full);
    uint64_t parent = 0;
    for (int j = 0; j < full; ++j) {
      const int32_t* t = tokens + (size_t)j * b;
      const uint64_t k = pkv_block_manager::chain(parent, t, b);
      keys.push_back(k);
      if (hits.size() == (size_t)j) {
        auto it = bm->cache.find(k);
        if (it != bm->cache.end() && it->second.parent == parent &&
            std::equal(it->second.tokens.begin(), it->second.tokens.end(), t))
          hits.push_back(it->second.block);
      }
      parent = k;
    }
  } catch (...) {
    return PKV_ERR_INVALID_ARG;
  }
  const long long need = ((long long)n_tokens + b - 1) / b - (long long)hits.size();
  long long revived = 0;
  for (int32_t h : hits) revived += bm->ref[h] == 0 ? 1 : 0;
  if (need > bm->allocatable() - revived) return PKV_ERR_NO_FREE_BLOCK;
  try {
    q.table.reserve(hits.size() + need);
    bm->cache.reserve(bm->cache.size() + (size_t)(full - (int)hits.size()));
  } catch (...) {
    return PKV_ERR_INVALID_ARG;
  }
  for (int32_t h : hits) {
    if (bm->ref[h] == 0) {
      bm->lru.erase(bm->lru_pos[h]);
      bm->ref[h] = 1;
    } else {
      bm->ref[h] += 1;
    }
    q.table.push_back(h);
  }
  for (long long i = 0; i < need; ++i) q.table.push_back(bm->alloc());
  for (int j = (int)hits.size(); j < full; ++j) {
    const uint64_t k = keys[j];
    if (bm->cache.count(k)) continue;
    const int32_t blk = q.table[j];
    pkv_block_manager::CacheEntry e;
    e.block = blk;
    e.parent = j == 0 ? 0 : keys[j - 1];
    e.tokens.assign(tokens + (size_t)j * b, tokens + (size_t)(j + 1) * b);
    bm->cache.emplace(k, std::move(e));
    bm->key_of[blk] = k;
    bm->cached[blk] = 1;
  }
  q.len = n_tokens;
  *cached_tokens_out = (int)hits.size() * b;
  return PKV_OK;
}

extern "C" int pkv_bm_num_cached(const pkv_block_manager* bm) {
  if (!bm) return PKV_ERR_INVALID_ARG;
  return (int)bm->cache.size();
}

// ---------------------------------------------------------------------------
// Groups for the shared-prefix (cascade) decode.  [lesson] "Sharing, and the
// reference counting it needs": sequences with a common prompt prefix hold
// the same physical blocks for it, so the groups can be read off the tables.
// ---------------------------------------------------------------------------

extern "C" int pkv_validate_cascade_groups(const int32_t* block_tables, int max_blocks_per_seq,
                                           const int32_t* context_lens, int num_seqs,
                                           int block_size, const int32_t* group_offsets,
                                           const int32_t* group_members, int num_members,
                                           const int32_t* group_prefix_blocks, int num_groups,
                                           int* bad_group_out) {
  if (bad_group_out) *bad_group_out = -1;
  if (num_seqs < 0 || max_blocks_per_seq < 1 || block_size < 1 || num_members < 0 ||
      num_groups < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_groups == 0) return PKV_OK;
  if (!group_offsets || !group_prefix_blocks || (num_members > 0 && !group_members) ||
      (num_seqs > 0 && (!block_tables || !context_lens)))
    return PKV_ERR_INVALID_ARG;
  std::vector<char> seen((size_t)num_seqs, 0);
  for (int z = 0; z < num_groups; ++z) {
    const int lo = group_offsets[z], hi = group_offsets[z + 1];
    const int pb = group_prefix_blocks[z];
    bool ok = lo >= 0 && hi >= lo && hi <= num_members && pb >= 0 && pb <= max_blocks_per_seq;
    const int32_t* ref_row = nullptr;
    for (int m = lo; ok && m < hi; ++m) {
      const int s = group_members[m];
      ok = s >= 0 && s < num_seqs && !seen[s] &&
           (long long)context_lens[s] >= (long long)pb * block_size;
      if (!ok) break;
      seen[s] = 1;
      const int32_t* row = block_tables + (size_t)s * max_blocks_per_seq;
      if (!ref_row) ref_row = row;
      ok = std::equal(row, row + pb, ref_row);
    }
    if (!ok) {
      if (bad_group_out) *bad_group_out = z;
      return PKV_ERR_INVALID_ARG;
    }
  }
  return PKV_OK;
}

extern "C" long long pkv_cascade_min_shared_tokens(int num_kv_heads, int head_dim,
                                                   int elem_bytes) {
  if (num_kv_heads < 1 || head_dim < 1 || elem_bytes < 1) return -1;
  const long long row = 2LL * num_kv_heads * head_dim * elem_bytes;   // K and V of a token
  return (PKV_CASCADE_MIN_SHARED_BYTES + row - 1) / row;
}

extern "C" int pkv_bm_export_cascade_groups(const pkv_block_manager* bm, const int* seqs, int n,
                                            int min_prefix_tokens, long long min_shared_tokens,
                                            int32_t* offsets_out, int32_t* members_out,
                                            int32_t* prefix_blocks_out, int* num_groups_out,
                                            int* num_members_out) {
  if (!bm || n < 0 || !num_groups_out || !num_members_out) return PKV_ERR_INVALID_ARG;
  if (n > 0 && (!seqs || !offsets_out || !members_out || !prefix_blocks_out))
    return PKV_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (!bm->seq_resident(seqs[i])) return PKV_ERR_INVALID_ARG;
  *num_groups_out = 0;
  *num_members_out = 0;
  if (n == 0) return PKV_OK;
  if (min_prefix_tokens < 0) min_prefix_tokens = PKV_CASCADE_MIN_PREFIX_TOKENS;
  if (min_shared_tokens < 0) min_shared_tokens = pkv_cascade_min_shared_tokens(8, 128, 2);
  const int b = bm->block_size;
  // Candidate groups: rows whose first table entry is the same block, in
  // order of first appearance; rows with no full block join none.
  std::unordered_map<int32_t, int> cand_of;
  std::vector<std::vector<int>> cand;
  for (int i = 0; i < n; ++i) {
    const auto& q = bm->seqs[seqs[i]];
    if (q.len < b) continue;
    auto it = cand_of.find(q.table[0]);
    if (it == cand_of.end()) {
      cand_of.emplace(q.table[0], (int)cand.size());
      cand.push_back({i});
    } else {
      cand[it->second].push_back(i);
    }
  }
  int groups = 0, members = 0;
  offsets_out[0] = 0;
  for (const auto& rows : cand) {
    if (rows.size() < 2) continue;
    // The prefix: leading entries every member shares, cut to the full
    // blocks of the shortest member (a partial block is still written).
    const auto& first = bm->seqs[seqs[rows[0]]];
    int pb = first.len / b;
    for (int r : rows) {
      const auto& q = bm->seqs[seqs[r]];
      pb = std::min(pb, q.len / b);
      int j = 0;
      while (j < pb && q.table[j] == first.table[j]) ++j;
      pb = j;
    }
    const long long prefix_tokens = (long long)pb * b;
    if (pb < 1 || prefix_tokens < min_prefix_tokens ||
        prefix_tokens * (long long)rows.size() < min_shared_tokens)
      continue;
    for (int r : rows) members_out[members++] = r;
    prefix_blocks_out[groups] = pb;
    offsets_out[++groups] = members;
  }
  *num_groups_out = groups;
  *num_members_out = members;
  return PKV_OK;
}
