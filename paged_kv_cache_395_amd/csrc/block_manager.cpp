// Host-side KV block manager: free list, per-sequence block lists, reference
// counts, copy-on-write.  Pure host code; produces the block tables and slots
// the device kernels consume.
//
// Pages: "PagedAttention: How vLLM Serves AI Like an Operating System" --
// blocks handed out on demand (section "The Magic: No Pre-allocation"), a
// logical-to-physical table per request and a free list (section
// "PagedAttention: Virtual Memory for KV Cache"), shared blocks with
// copy-on-write for parallel sampling and a common system prompt (section
// "Copy-on-Write: Sharing KV Cache"); "vLLM Architecture and PagedAttention -
// Interactive Visualization" (Page Table Visualization): a finished
// sequence's pages return to the pool at once.

#include "bm_internal.h"

#include <unordered_set>

using pa::fail;

namespace pa {

int64_t append_need(const pa_bm* bm, const int64_t* seqs, int32_t n, int64_t* cows) {
  // Decide, without changing anything, how many blocks a batch of appends
  // takes and how many of them are copy-on-write.  Per sequence track the
  // token count and whether its last block is already private; per shared
  // block track its count as earlier writers in the batch leave it.
  struct SimSeq {
    int32_t tokens;
    bool last_private;
  };
  std::unordered_map<int64_t, SimSeq> sim;
  std::unordered_map<int32_t, int32_t> sim_ref;
  int64_t need = 0, nc = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return -fail(PA_ENOENT, "unknown sequence %lld", (long long)seqs[i]);
    if (it->second.swapped) return -fail(PA_EINVAL, "sequence %lld is swapped out", (long long)seqs[i]);
    auto si = sim.find(seqs[i]);
    SimSeq st = si == sim.end() ? SimSeq{it->second.tokens, false} : si->second;
    if (st.tokens == INT32_MAX) return -fail(PA_EINVAL, "sequence too long");
    if (st.tokens % bm->bs == 0) {
      ++need;
      st.last_private = true;
    } else if (!st.last_private) {
      const int32_t last = it->second.blocks.back();
      auto ri = sim_ref.find(last);
      const int32_t r = ri == sim_ref.end() ? bm->ref[size_t(last)] : ri->second;
      if (r > 1) {
        ++need;
        ++nc;
        sim_ref[last] = r - 1;
      }
      st.last_private = true;
    }
    st.tokens += 1;
    sim[seqs[i]] = st;
  }
  if (cows) *cows = nc;
  return need;
}

}  // namespace pa

namespace {

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

// Validate a list of sequences for a swap: all known, none listed twice,
// each in the expected residence.
pa_status_t check_swap_list(const pa_bm* bm, const int64_t* seqs, int32_t n, bool want_swapped, int64_t* blocks) {
  if (n < 0 || (n > 0 && !seqs)) return fail(PA_EINVAL, "bad arguments");
  std::unordered_set<int64_t> seen;
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return fail(PA_ENOENT, "unknown sequence %lld", (long long)seqs[i]);
    if (!seen.insert(seqs[i]).second) return fail(PA_EINVAL, "sequence %lld listed twice", (long long)seqs[i]);
    if (it->second.swapped != want_swapped)
      return fail(PA_EINVAL, "sequence %lld is %s", (long long)seqs[i],
                  want_swapped ? "not swapped out" : "already swapped out");
    total += int64_t(it->second.blocks.size());
  }
  *blocks = total;
  return PA_OK;
}

// Key of a full block: a hash of the prefix hash before it and its token
// ids (FNV-1a 64 over their bytes, then the SplitMix64 finalizer to spread
// the bits).  A match is confirmed against the stored parent hash and token
// ids, so only a collision of whole-prefix hashes could mislead it.
uint64_t block_key(uint64_t parent, const int32_t* tok, int32_t bs) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&h](uint64_t x, int bytes) {
    for (int i = 0; i < bytes; ++i) {
      h ^= (x >> (8 * i)) & 0xffu;
      h *= 1099511628211ull;
    }
  };
  mix(parent, 8);
  for (int i = 0; i < bs; ++i) mix(uint32_t(tok[i]), 4);
  h ^= h >> 30;
  h *= 0xbf58476d1ce4e5b9ull;
  h ^= h >> 27;
  h *= 0x94d049bb133111ebull;
  h ^= h >> 31;
  return h;
}

// The cached block holding exactly this (parent, tokens), or -1.
int32_t lookup(const pa_bm* bm, uint64_t k, uint64_t parent, const int32_t* tok) {
  auto it = bm->cached.find(k);
  if (it == bm->cached.end()) return -1;
  const int32_t b = it->second;
  if (bm->parent_key[size_t(b)] != parent) return -1;
  for (int i = 0; i < bm->bs; ++i)
    if (bm->key_tokens[size_t(b) * bm->bs + i] != tok[i]) return -1;
  return b;
}

// Distinct blocks among the listed sequences' block lists.
int64_t distinct_blocks(const pa_bm* bm, const int64_t* seqs, int32_t n) {
  std::unordered_set<int32_t> d;
  for (int32_t i = 0; i < n; ++i)
    for (int32_t b : bm->seqs.find(seqs[i])->second.blocks) d.insert(b);
  return int64_t(d.size());
}

}  // namespace

namespace pa {

int64_t prefix_probe(const pa_bm* bm, const int32_t* tokens, int32_t num_tokens, std::vector<int32_t>* hits,
                     std::vector<uint64_t>* keys, std::vector<uint64_t>* parents) {
  const int32_t full = num_tokens / bm->bs;
  keys->assign(size_t(full), 0);
  parents->assign(size_t(full), 0);
  hits->clear();
  uint64_t parent = 0;
  bool hitting = true;
  int64_t claimed = 0;
  for (int32_t i = 0; i < full; ++i) {
    const int32_t* tok = tokens + int64_t(i) * bm->bs;
    (*parents)[size_t(i)] = parent;
    (*keys)[size_t(i)] = block_key(parent, tok, bm->bs);
    if (hitting) {
      const int32_t b = lookup(bm, (*keys)[size_t(i)], parent, tok);
      if (b >= 0) {
        hits->push_back(b);
        claimed += bm->in_lru[size_t(b)];
      } else {
        hitting = false;
      }
    }
    parent = (*keys)[size_t(i)];
  }
  return claimed;
}

}  // namespace pa

extern "C" {

pa_bm_t* pa_bm_create(int64_t num_blocks, int32_t block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || num_blocks > INT32_MAX || !(block_size == 16 || block_size == 32 || block_size == 64)) {
    fail(PA_EINVAL, "pa_bm_create: num_blocks must be in [1, 2^31) and block_size 16, 32 or 64");
    return nullptr;
  }
  pa_bm* bm = new (std::nothrow) pa_bm;
  if (!bm) {
    fail(PA_EINVAL, "pa_bm_create: out of host memory");
    return nullptr;
  }
  bm->num_blocks = num_blocks;
  bm->bs = block_size;
  bm->ref.assign(size_t(num_blocks), 0);
  if (free_order) {
    std::vector<char> seen(size_t(num_blocks), 0);
    for (int64_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[size_t(b)]) {
        delete bm;
        fail(PA_EINVAL, "pa_bm_create: free_order is not a permutation of the pool");
        return nullptr;
      }
      seen[size_t(b)] = 1;
      bm->free_q.push_back(b);
    }
  } else {
    for (int64_t i = 0; i < num_blocks; ++i) bm->free_q.push_back(int32_t(i));
  }
  return bm;
}

void pa_bm_destroy(pa_bm_t* bm) { delete bm; }

pa_status_t pa_bm_add_seq(pa_bm_t* bm, int64_t seq, int32_t num_tokens) {
  if (!bm) return fail(PA_EINVAL, "null block manager");
  if (num_tokens < 0) return fail(PA_EINVAL, "negative length");
  if (bm->seqs.count(seq)) return fail(PA_EINVAL, "sequence %lld already exists", (long long)seq);
  const int64_t need = blocks_for(num_tokens, bm->bs);
  if (need > bm->available())
    return fail(PA_ENOSPC, "need %lld blocks, %lld free", (long long)need, (long long)bm->available());
  Seq s;
  s.tokens = num_tokens;
  s.blocks.reserve(size_t(need));
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
  bm->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

pa_status_t pa_bm_add_seq_with_prefix(pa_bm_t* bm, int64_t seq, int64_t prefix_seq, int32_t prefix_tokens,
                                      int32_t tail_tokens) {
  if (!bm) return fail(PA_EINVAL, "null block manager");
  if (bm->seqs.count(seq)) return fail(PA_EINVAL, "sequence %lld already exists", (long long)seq);
  auto it = bm->seqs.find(prefix_seq);
  if (it == bm->seqs.end()) return fail(PA_ENOENT, "unknown prefix sequence %lld", (long long)prefix_seq);
  if (it->second.swapped) return fail(PA_EINVAL, "prefix sequence %lld is swapped out", (long long)prefix_seq);
  if (prefix_tokens < 0 || prefix_tokens % bm->bs != 0 || prefix_tokens > it->second.tokens || tail_tokens < 0)
    return fail(PA_EINVAL, "a shared prefix is a whole number of blocks inside the prefix sequence");
  const int64_t need = blocks_for(tail_tokens, bm->bs);
  if (need > bm->available())
    return fail(PA_ENOSPC, "need %lld blocks, %lld free", (long long)need, (long long)bm->available());
  Seq s;
  s.tokens = prefix_tokens + tail_tokens;
  const int32_t shared = prefix_tokens / bm->bs;
  s.blocks.assign(it->second.blocks.begin(), it->second.blocks.begin() + shared);
  for (int32_t b : s.blocks) ++bm->ref[size_t(b)];
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
  bm->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

pa_status_t pa_bm_fork(pa_bm_t* bm, int64_t parent, int64_t child) {
  if (!bm) return fail(PA_EINVAL, "null block manager");
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return fail(PA_ENOENT, "unknown parent %lld", (long long)parent);
  if (it->second.swapped) return fail(PA_EINVAL, "parent %lld is swapped out", (long long)parent);
  if (bm->seqs.count(child)) return fail(PA_EINVAL, "sequence %lld already exists", (long long)child);
  Seq s = it->second;
  for (int32_t b : s.blocks) ++bm->ref[size_t(b)];
  bm->seqs.emplace(child, std::move(s));
  return PA_OK;
}

pa_status_t pa_bm_free_seq(pa_bm_t* bm, int64_t seq) {
  if (!bm) return fail(PA_EINVAL, "null block manager");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PA_ENOENT, "unknown sequence %lld", (long long)seq);
  const std::vector<int32_t>& bl = it->second.blocks;
  if (it->second.swapped) {
    for (int32_t h : bl) bm->drop_host(h);
  } else if (bm->prefix_cache) {
    // deepest block first, so a cached prefix is evicted from its end
    for (auto b = bl.rbegin(); b != bl.rend(); ++b) bm->drop(*b);
  } else {
    for (int32_t b : bl) bm->drop(b);
  }
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status_t pa_bm_append_tokens(pa_bm_t* bm, const int64_t* seqs, int32_t n, int64_t* slots, int64_t* cow_pairs,
                                int32_t* num_cow) {
  if (!bm) return fail(PA_EINVAL, "null block manager");
  if (n < 0 || (n > 0 && (!seqs || !slots))) return fail(PA_EINVAL, "bad arguments");
  if (num_cow) *num_cow = 0;
  int64_t cows = 0;
  const int64_t need = pa::append_need(bm, seqs, n, &cows);
  if (need < 0) return pa_status_t(-need);
  if (need > bm->available())
    return fail(PA_ENOSPC, "need %lld blocks, %lld free", (long long)need, (long long)bm->available());
  if (cows > 0 && !cow_pairs) return fail(PA_EINVAL, "copy-on-write needed but cow_pairs is NULL");
  // Pass 2: apply; cannot fail.
  int32_t nc = 0;
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = bm->seqs.find(seqs[i])->second;
    const int32_t pos = s.tokens;
    if (pos % bm->bs == 0) {
      s.blocks.push_back(bm->take());
    } else {
      const int32_t last = s.blocks.back();
      if (bm->ref[size_t(last)] > 1) {
        const int32_t fresh = bm->take();
        --bm->ref[size_t(last)];
        s.blocks.back() = fresh;
        cow_pairs[2 * nc] = last;
        cow_pairs[2 * nc + 1] = fresh;
        ++nc;
      }
    }
    slots[i] = int64_t(s.blocks[size_t(pos / bm->bs)]) * bm->bs + pos % bm->bs;
    s.tokens = pos + 1;
  }
  if (num_cow) *num_cow = nc;
  return PA_OK;
}

pa_status_t pa_bm_block_table(const pa_bm_t* bm, const int64_t* seqs, int32_t n, int32_t max_blocks, int32_t pad_id,
                              int32_t* table, int32_t* context_lens) {
  if (!bm) return fail(PA_EINVAL, "null block manager");
  if (n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !table || !context_lens))) return fail(PA_EINVAL, "bad arguments");
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return fail(PA_ENOENT, "unknown sequence %lld", (long long)seqs[i]);
    if (it->second.swapped) return fail(PA_EINVAL, "sequence %lld is swapped out", (long long)seqs[i]);
    if (int64_t(it->second.blocks.size()) > max_blocks)
      return fail(PA_EINVAL, "sequence %lld holds %zu blocks > max_blocks %d", (long long)seqs[i],
                  it->second.blocks.size(), max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = table + int64_t(i) * max_blocks;
    const size_t nb = s.blocks.size();
    for (size_t j = 0; j < nb; ++j) row[j] = s.blocks[j];
    for (int64_t j = int64_t(nb); j < max_blocks; ++j) row[j] = pad_id;
    context_lens[i] = s.tokens;
  }
  return PA_OK;
}

pa_status_t pa_bm_set_host_pool(pa_bm_t* bm, int64_t num_host_blocks) {
  if (!bm) return fail(PA_EINVAL, "null block manager");
  if (num_host_blocks < 0 || num_host_blocks > INT32_MAX) return fail(PA_EINVAL, "num_host_blocks out of range");
  if (bm->num_host_blocks != 0) return fail(PA_EINVAL, "the host pool is already set");
  bm->num_host_blocks = num_host_blocks;
  bm->host_ref.assign(size_t(num_host_blocks), 0);
  for (int64_t i = 0; i < num_host_blocks; ++i) bm->host_free.push_back(int32_t(i));
  return PA_OK;
}

pa_status_t pa_bm_swap_out(pa_bm_t* bm, const int64_t* seqs, int32_t n, int64_t* pairs, int32_t* num_pairs) {
  if (!bm) return fail(PA_EINVAL, "null block manager");
  if (num_pairs) *num_pairs = 0;
  int64_t total = 0;
  pa_status_t st = check_swap_list(bm, seqs, n, false, &total);
  if (st != PA_OK) return st;
  if (total > 0 && !pairs) return fail(PA_EINVAL, "pairs is NULL");
  const int64_t need = distinct_blocks(bm, seqs, n);
  if (need > int64_t(bm->host_free.size()))
    return fail(PA_ENOSPC, "need %lld host blocks, %zu free", (long long)need, bm->host_free.size());
  std::unordered_map<int32_t, int32_t> moved;  // device block -> host block, within this call
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = bm->seqs.find(seqs[i])->second;
    for (int32_t& b : s.blocks) {
      auto mi = moved.find(b);
      int32_t h;
      if (mi == moved.end()) {
        h = bm->take_host();
        moved.emplace(b, h);
        pairs[2 * np] = b;
        pairs[2 * np + 1] = h;
        ++np;
      } else {
        h = mi->second;
        ++bm->host_ref[size_t(h)];
      }
      bm->drop(b);
      b = h;
    }
    s.swapped = true;
  }
  if (num_pairs) *num_pairs = np;
  return PA_OK;
}

pa_status_t pa_bm_swap_in(pa_bm_t* bm, const int64_t* seqs, int32_t n, int64_t* pairs, int32_t* num_pairs) {
  if (!bm) return fail(PA_EINVAL, "null block manager");
  if (num_pairs) *num_pairs = 0;
  int64_t total = 0;
  pa_status_t st = check_swap_list(bm, seqs, n, true, &total);
  if (st != PA_OK) return st;
  if (total > 0 && !pairs) return fail(PA_EINVAL, "pairs is NULL");
  const int64_t need = distinct_blocks(bm, seqs, n);
  if (need > bm->available())
    return fail(PA_ENOSPC, "need %lld blocks, %lld free", (long long)need, (long long)bm->available());
  std::unordered_map<int32_t, int32_t> moved;  // host block -> device block, within this call
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = bm->seqs.find(seqs[i])->second;
    for (int32_t& h : s.blocks) {
      auto mi = moved.find(h);
      int32_t b;
      if (mi == moved.end()) {
        b = bm->take();
        moved.emplace(h, b);
        pairs[2 * np] = h;
        pairs[2 * np + 1] = b;
        ++np;
      } else {
        b = mi->second;
        ++bm->ref[size_t(b)];
      }
      bm->drop_host(h);
      h = b;
    }
    s.swapped = false;
  }
  if (num_pairs) *num_pairs = np;
  return PA_OK;
}

int32_t pa_bm_is_swapped(const pa_bm_t* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : int32_t(it->second.swapped);
}

int64_t pa_bm_num_free_host(const pa_bm_t* bm) { return bm ? int64_t(bm->host_free.size()) : -1; }

int32_t pa_bm_host_refcount(const pa_bm_t* bm, int64_t block) {
  if (!bm || block < 0 || block >= bm->num_host_blocks) return -1;
  return bm->host_ref[size_t(block)];
}

pa_status_t pa_bm_enable_prefix_cache(pa_bm_t* bm) {
  if (!bm) return fail(PA_EINVAL, "null block manager");
  if (bm->prefix_cache) return fail(PA_EINVAL, "prefix caching is already on");
  if (!bm->seqs.empty()) return fail(PA_EINVAL, "turn prefix caching on before adding sequences");
  const size_t nb = size_t(bm->num_blocks);
  bm->prefix_cache = true;
  bm->key.assign(nb, 0);
  bm->parent_key.assign(nb, 0);
  bm->key_tokens.assign(nb * size_t(bm->bs), 0);
  bm->keyed.assign(nb, 0);
  bm->in_lru.assign(nb, 0);
  bm->lru_pos.assign(nb, bm->lru.end());
  return PA_OK;
}


pa_status_t pa_bm_add_seq_tokens(pa_bm_t* bm, int64_t seq, const int32_t* tokens, int32_t num_tokens,
                                 int32_t* cached_tokens) {
  if (!bm) return fail(PA_EINVAL, "null block manager");
  if (!bm->prefix_cache) return fail(PA_EINVAL, "prefix caching is off (pa_bm_enable_prefix_cache)");
  if (num_tokens < 0 || (num_tokens > 0 && !tokens)) return fail(PA_EINVAL, "bad arguments");
  if (bm->seqs.count(seq)) return fail(PA_EINVAL, "sequence %lld already exists", (long long)seq);
  const int32_t full = num_tokens / bm->bs;
  const int64_t total = blocks_for(num_tokens, bm->bs);
  // the leading run of full blocks already cached
  std::vector<uint64_t> keys, parents;
  std::vector<int32_t> hits;
  const int64_t from_lru = pa::prefix_probe(bm, tokens, num_tokens, &hits, &keys, &parents);
  const int64_t need = total - int64_t(hits.size());
  if (need > bm->available() - from_lru)
    return fail(PA_ENOSPC, "need %lld blocks, %lld free", (long long)need, (long long)(bm->available() - from_lru));
  Seq s;
  s.tokens = num_tokens;
  s.blocks.reserve(size_t(total));
  for (int32_t b : hits) {
    if (bm->in_lru[size_t(b)]) bm->lru_remove(b);
    ++bm->ref[size_t(b)];
    s.blocks.push_back(b);
  }
  for (int64_t i = int64_t(hits.size()); i < total; ++i) {
    const int32_t b = bm->take();
    s.blocks.push_back(b);
    if (i < full) {  // a full prompt block: key it (the caller writes its tokens this step)
      const uint64_t k = keys[size_t(i)];
      auto it = bm->cached.find(k);
      if (it != bm->cached.end()) {  // a stale entry for the same prefix: the new block replaces it
        const int32_t old = it->second;
        bm->keyed[size_t(old)] = 0;
        if (bm->in_lru[size_t(old)]) {
          bm->lru_remove(old);
          bm->free_q.push_back(old);
        }
      }
      bm->cached[k] = b;
      bm->key[size_t(b)] = k;
      bm->parent_key[size_t(b)] = parents[size_t(i)];
      for (int t = 0; t < bm->bs; ++t) bm->key_tokens[size_t(b) * bm->bs + t] = tokens[i * bm->bs + t];
      bm->keyed[size_t(b)] = 1;
    }
  }
  bm->seqs.emplace(seq, std::move(s));
  if (cached_tokens) *cached_tokens = int32_t(hits.size()) * bm->bs;
  return PA_OK;
}

int64_t pa_bm_num_cached_free(const pa_bm_t* bm) { return bm ? int64_t(bm->lru.size()) : -1; }

int64_t pa_bm_num_free(const pa_bm_t* bm) { return bm ? bm->available() : -1; }

int32_t pa_bm_refcount(const pa_bm_t* bm, int64_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[size_t(block)];
}

double pa_bm_usage(const pa_bm_t* bm) {
  if (!bm) return -1.0;
  return double(bm->num_blocks - bm->available()) / double(bm->num_blocks);
}

int32_t pa_bm_num_tokens(const pa_bm_t* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.tokens;
}

int64_t pa_bm_free_list(const pa_bm_t* bm, int32_t* out, int64_t cap) {
  if (!bm) return -1;
  int64_t i = 0;
  for (int32_t b : bm->free_q) {
    if (i < cap && out) out[i] = b;
    ++i;
  }
  return i;
}

}  // extern "C"
