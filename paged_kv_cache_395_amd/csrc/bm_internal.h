// Host block manager state, shared by the block manager's entry points and
// the step scheduler built on it.  Host code only.
#ifndef PA_BM_INTERNAL_H
#define PA_BM_INTERNAL_H

#include <stdint.h>

#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

namespace pa {
constexpr int32_t kBlockTokensHost = 16;
}

struct Seq {
  std::vector<int32_t> blocks;  // device block ids; host block ids while swapped out
  int32_t tokens = 0;
  bool swapped = false;
};

struct pa_bm {
  int64_t num_blocks = 0;
  std::vector<int32_t> ref;
  std::deque<int32_t> free_q;  // head = next block handed out, tail = most recently released
  std::unordered_map<int64_t, Seq> seqs;
  // host (swap) pool: same queue discipline, its own ids
  int64_t num_host_blocks = 0;
  std::vector<int32_t> host_ref;
  std::deque<int32_t> host_free;

  int32_t take() {
    const int32_t b = free_q.front();
    free_q.pop_front();
    ref[size_t(b)] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--ref[size_t(b)] == 0) free_q.push_back(b);
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
}  // namespace pa

#endif
