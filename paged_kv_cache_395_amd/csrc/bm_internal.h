// Host block manager state, shared by the block manager's entry points and
// the step scheduler built on it.  Host code only.
#ifndef PA_BM_INTERNAL_H
#define PA_BM_INTERNAL_H

#include <stdint.h>

#include <deque>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

struct Seq {
  std::vector<int32_t> blocks;  // device block ids; host block ids while swapped out
  int32_t tokens = 0;
  bool swapped = false;
};

struct pa_bm {
  int64_t num_blocks = 0;
  int32_t bs = 16;  // tokens per block: 16, 32 or 64
  std::vector<int32_t> ref;
  std::deque<int32_t> free_q;  // head = next block handed out, tail = most recently released
  std::unordered_map<int64_t, Seq> seqs;
  // host (swap) pool: same queue discipline, its own ids
  int64_t num_host_blocks = 0;
  std::vector<int32_t> host_ref;
  std::deque<int32_t> host_free;
  // prefix cache: full prompt blocks keyed by a hash of their whole prefix;
  // a keyed block whose count drops to zero waits in `lru` (head = evicted
  // first) and can be claimed again until it is evicted
  bool prefix_cache = false;
  std::unordered_map<uint64_t, int32_t> cached;  // prefix hash -> block
  std::vector<uint64_t> key;                     // per block: its prefix hash (valid when keyed)
  std::vector<uint64_t> parent_key;              // per block: the hash of the prefix before it
  std::vector<int32_t> key_tokens;               // per block: its block_size token ids
  std::vector<char> keyed, in_lru;
  std::list<int32_t> lru;
  std::vector<std::list<int32_t>::iterator> lru_pos;

  int64_t available() const { return int64_t(free_q.size()) + int64_t(lru.size()); }
  void unkey(int32_t b) {
    cached.erase(key[size_t(b)]);
    keyed[size_t(b)] = 0;
  }
  void lru_remove(int32_t b) {
    lru.erase(lru_pos[size_t(b)]);
    in_lru[size_t(b)] = 0;
  }
  int32_t take() {
    int32_t b;
    if (!free_q.empty()) {
      b = free_q.front();
      free_q.pop_front();
    } else {  // evict the least recently released cached block
      b = lru.front();
      lru_remove(b);
      unkey(b);
    }
    ref[size_t(b)] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--ref[size_t(b)] != 0) return;
    if (prefix_cache && keyed[size_t(b)]) {
      lru_pos[size_t(b)] = lru.insert(lru.end(), b);
      in_lru[size_t(b)] = 1;
    } else {
      free_q.push_back(b);
    }
  }
  int32_t take_host() {
    const int32_t h = host_free.front();
    host_free.pop_front();
    host_ref[size_t(h)] = 1;
    return h;
  }
  void drop_host(int32_t h) {
    if (--host_ref[size_t(h)] == 0) host_free.push_back(h);
  }
};

namespace pa {
// Blocks (fresh or copy-on-write) that appending one token to each of
// seqs[0..n) would take; the copy-on-write count goes to *cows.  Returns
// -status (after recording the message) for an unknown or swapped-out
// sequence.  Changes nothing.
int64_t append_need(const pa_bm* bm, const int64_t* seqs, int32_t n, int64_t* cows);
// The leading run of cached full blocks of a token list (into *hits), with
// every full block's prefix key and the key before it; returns how many of
// the hits sit in the evictable list.  Prefix caching must be on.  Changes
// nothing.
int64_t prefix_probe(const pa_bm* bm, const int32_t* tokens, int32_t num_tokens, std::vector<int32_t>* hits,
                     std::vector<uint64_t>* keys, std::vector<uint64_t>* parents);
}  // namespace pa

#endif
