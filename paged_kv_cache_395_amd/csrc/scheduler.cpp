// Continuous-batching step scheduler on top of the host block manager.
//
// Pages: "PagedAttention: How vLLM Serves AI Like an Operating System" --
// section "Continuous Batching: The Other Half" (a request leaves the batch
// as soon as it is done and a waiting one takes its place at the next step;
// with paged memory only the block table changes) and section "vLLM
// Architecture" (the scheduler asks the cache manager how many blocks are
// free, picks the requests of each step, and preempts low-priority requests
// by moving their blocks to CPU memory); "vLLM Architecture and
// PagedAttention - Interactive Visualization" (Continuous Batching).
//
// Policy (the pages name the pieces, not the rules; these are the plainest
// ones that fit them):
//   priority   = arrival order (earlier submit first);
//   rows       = a fixed set of batch rows; a request keeps its row while it
//                runs, a new or swapped-in one takes the lowest free row;
//   each step  = retire finished requests; reserve the blocks every running
//                request's next token needs, preempting the lowest-priority
//                running request while they do not fit (swap out to the host
//                pool, or -- when the host pool is full -- drop its blocks and
//                requeue it to be recomputed); swap back in, highest priority
//                first; admit waiting requests only when nothing is swapped
//                out; append one token to every request that was running
//                before the admissions.

#include <algorithm>
#include <unordered_set>

#include "bm_internal.h"

using pa::fail;

namespace {

struct Req {
  int64_t seq;
  int64_t arrival;
  int32_t prompt;  // tokens written when admitted
  int32_t total;   // the request is done once its sequence holds this many tokens
  int32_t row;
  std::vector<int32_t> ids;  // prompt token ids, when given (admission then reuses cached prefix blocks)
};

void insert_by_arrival(std::vector<Req>& v, const Req& r) {
  auto pos = std::upper_bound(v.begin(), v.end(), r.arrival,
                              [](int64_t a, const Req& x) { return a < x.arrival; });
  v.insert(pos, r);
}

int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

}  // namespace

struct pa_sched {
  pa_bm* bm = nullptr;
  int32_t max_rows = 0, max_blocks = 0, max_batched_tokens = 0;
  int64_t next_arrival = 0;
  std::vector<Req> waiting, running, swapped;  // each sorted by arrival
  std::unordered_set<int64_t> known;
  std::vector<int64_t> row_seq;
  // outputs of the last step
  std::vector<int64_t> slots, swap_out, swap_in, cow, finished;
  std::vector<int32_t> rows, positions, ctx, patches;
  std::vector<int64_t> scratch_pairs;
  pa_sched_out_t out{};

  int32_t free_row() const {
    for (int32_t r = 0; r < max_rows; ++r)
      if (row_seq[size_t(r)] < 0) return r;
    return -1;
  }
  const Seq& seq_of(int64_t id) const { return bm->seqs.find(id)->second; }
  int64_t free_blocks() const { return bm->available(); }
  int64_t running_need() const {
    std::vector<int64_t> ids;
    ids.reserve(running.size());
    for (const Req& r : running) ids.push_back(r.seq);
    return pa::append_need(bm, ids.data(), int32_t(ids.size()), nullptr);
  }
};

extern "C" {

pa_sched_t* pa_sched_create(pa_bm_t* bm, int32_t max_rows, int32_t max_blocks_per_seq, int32_t max_batched_tokens) {
  if (!bm || max_rows <= 0 || max_blocks_per_seq <= 0 || max_batched_tokens <= 0) {
    fail(PA_EINVAL, "pa_sched_create: need a block manager and positive sizes");
    return nullptr;
  }
  pa_sched* s = new (std::nothrow) pa_sched;
  if (!s) {
    fail(PA_EINVAL, "pa_sched_create: out of host memory");
    return nullptr;
  }
  s->bm = bm;
  s->max_rows = max_rows;
  s->max_blocks = max_blocks_per_seq;
  s->max_batched_tokens = max_batched_tokens;
  s->row_seq.assign(size_t(max_rows), -1);
  s->ctx.assign(size_t(max_rows), 0);
  return s;
}

void pa_sched_destroy(pa_sched_t* s) { delete s; }

pa_status_t pa_sched_submit(pa_sched_t* s, int64_t seq, int32_t prompt_tokens, int32_t total_tokens) {
  return pa_sched_submit_tokens(s, seq, nullptr, prompt_tokens, total_tokens);
}

pa_status_t pa_sched_submit_tokens(pa_sched_t* s, int64_t seq, const int32_t* prompt_ids, int32_t prompt_tokens,
                                   int32_t total_tokens) {
  if (!s) return fail(PA_EINVAL, "null scheduler");
  if (seq < 0) return fail(PA_EINVAL, "request ids must be >= 0");
  if (prompt_tokens < 1 || total_tokens < prompt_tokens)
    return fail(PA_EINVAL, "need 1 <= prompt_tokens <= total_tokens");
  const int64_t nb = blocks_for(total_tokens, s->bm->bs);
  if (nb > s->max_blocks || nb > s->bm->num_blocks)
    return fail(PA_EINVAL, "a request of %d tokens can never fit (%lld blocks)", total_tokens, (long long)nb);
  if (s->known.count(seq) || s->bm->seqs.count(seq))
    return fail(PA_EINVAL, "sequence %lld already exists", (long long)seq);
  if (prompt_ids && !s->bm->prefix_cache) return fail(PA_EINVAL, "token ids need prefix caching on");
  s->known.insert(seq);
  Req r{seq, s->next_arrival++, prompt_tokens, total_tokens, -1, {}};
  if (prompt_ids) r.ids.assign(prompt_ids, prompt_ids + prompt_tokens);
  s->waiting.push_back(std::move(r));
  return PA_OK;
}

pa_status_t pa_sched_step(pa_sched_t* s, pa_sched_out_t* out) {
  if (!s || !out) return fail(PA_EINVAL, "null argument");
  pa_bm* bm = s->bm;
  // the requests it runs or has swapped out must still be in the block
  // manager (checked before anything changes)
  for (const std::vector<Req>* v : {&s->running, &s->swapped})
    for (const Req& r : *v)
      if (!bm->seqs.count(r.seq))
        return fail(PA_ENOENT, "request %lld was removed from the block manager behind the scheduler",
                    (long long)r.seq);
  s->slots.clear();
  s->rows.clear();
  s->positions.clear();
  s->swap_out.clear();
  s->swap_in.clear();
  s->cow.clear();
  s->patches.clear();
  s->finished.clear();
  pa_sched_out_t o{};

  // 1. retire requests that reached their length
  {
    std::vector<Req> keep;
    keep.reserve(s->running.size());
    for (const Req& r : s->running) {
      if (s->seq_of(r.seq).tokens >= r.total) {
        pa_bm_free_seq(bm, r.seq);
        s->row_seq[size_t(r.row)] = -1;
        s->finished.push_back(r.seq);
        s->known.erase(r.seq);
      } else {
        keep.push_back(r);
      }
    }
    s->running.swap(keep);
  }

  // 2. reserve every running request's next token; preempt from the lowest priority while short
  std::unordered_set<int64_t> preempted;
  int64_t reserved = s->running_need();
  if (reserved < 0) return pa_status_t(-reserved);
  while (reserved > s->free_blocks() && !s->running.empty()) {
    Req v = s->running.back();
    s->running.pop_back();
    s->row_seq[size_t(v.row)] = -1;
    v.row = -1;
    preempted.insert(v.seq);
    const Seq& sq = s->seq_of(v.seq);
    if (int64_t(sq.blocks.size()) <= int64_t(bm->host_free.size())) {
      s->scratch_pairs.resize(2 * sq.blocks.size() + 2);
      int32_t np = 0;
      pa_status_t st = pa_bm_swap_out(bm, &v.seq, 1, s->scratch_pairs.data(), &np);
      if (st != PA_OK) return st;
      s->swap_out.insert(s->swap_out.end(), s->scratch_pairs.begin(), s->scratch_pairs.begin() + 2 * np);
      insert_by_arrival(s->swapped, v);
      ++o.num_preempted_swap;
    } else {
      v.prompt = sq.tokens;  // recomputed from its tokens so far when readmitted (by count: no ids)
      v.ids.clear();
      pa_bm_free_seq(bm, v.seq);
      insert_by_arrival(s->waiting, v);
      ++o.num_preempted_recompute;
    }
    reserved = s->running_need();
    if (reserved < 0) return pa_status_t(-reserved);
  }

  // 3. swap back in, highest priority first, while a row and the blocks are there
  while (!s->swapped.empty()) {
    Req r = s->swapped.front();
    if (preempted.count(r.seq)) break;
    const int32_t row = s->free_row();
    if (row < 0) break;
    const Seq& sq = s->seq_of(r.seq);
    const int64_t nb = int64_t(sq.blocks.size());
    const int64_t grow = sq.tokens % bm->bs == 0 ? 1 : 0;
    if (nb + grow + reserved > s->free_blocks()) break;
    s->scratch_pairs.resize(2 * size_t(nb) + 2);
    int32_t np = 0;
    pa_status_t st = pa_bm_swap_in(bm, &r.seq, 1, s->scratch_pairs.data(), &np);
    if (st != PA_OK) return st;
    s->swap_in.insert(s->swap_in.end(), s->scratch_pairs.begin(), s->scratch_pairs.begin() + 2 * np);
    reserved += grow;
    r.row = row;
    s->row_seq[size_t(row)] = r.seq;
    const Seq& now = s->seq_of(r.seq);
    for (size_t j = 0; j < now.blocks.size(); ++j) {
      s->patches.push_back(row);
      s->patches.push_back(int32_t(j));
      s->patches.push_back(now.blocks[j]);
    }
    insert_by_arrival(s->running, r);
    s->swapped.erase(s->swapped.begin());
    ++o.num_swapped_in;
  }

  // 4. admit waiting requests (first come, first served) while nothing is swapped out
  std::unordered_set<int64_t> admitted;
  if (s->swapped.empty()) {
    int64_t budget = int64_t(s->max_batched_tokens) - int64_t(s->running.size());
    std::vector<int32_t> hits;
    std::vector<uint64_t> keys, parents;
    while (!s->waiting.empty()) {
      Req& r = s->waiting.front();
      const int32_t row = s->free_row();
      if (row < 0) break;
      // blocks the admission takes: fresh ones, plus cached ones it claims back from the evictable list
      int64_t take = blocks_for(r.prompt, bm->bs), write_from = 0;
      const bool by_ids = !r.ids.empty();
      if (by_ids) {
        const int64_t claimed = pa::prefix_probe(bm, r.ids.data(), r.prompt, &hits, &keys, &parents);
        take = take - int64_t(hits.size()) + claimed;
      }
      if (take + reserved > s->free_blocks()) break;
      if (!admitted.empty() && r.prompt > budget) break;  // the first admission of a step is always allowed
      pa_status_t st;
      if (by_ids) {
        int32_t cached = 0;
        st = pa_bm_add_seq_tokens(bm, r.seq, r.ids.data(), r.prompt, &cached);
        write_from = cached;
        o.num_cached_tokens += cached;
      } else {
        st = pa_bm_add_seq(bm, r.seq, r.prompt);
      }
      if (st != PA_OK) return st;
      const Seq& sq = s->seq_of(r.seq);
      for (int64_t j = 0; j < write_from / bm->bs; ++j) {  // cached blocks get no token write: patch the table
        s->patches.push_back(row);
        s->patches.push_back(int32_t(j));
        s->patches.push_back(sq.blocks[size_t(j)]);
      }
      for (int32_t p = int32_t(write_from); p < r.prompt; ++p) {
        s->slots.push_back(int64_t(sq.blocks[size_t(p / bm->bs)]) * bm->bs + p % bm->bs);
        s->rows.push_back(row);
        s->positions.push_back(p);
      }
      budget -= r.prompt;
      r.row = row;
      s->row_seq[size_t(row)] = r.seq;
      admitted.insert(r.seq);
      Req moved = std::move(r);
      moved.ids.clear();  // only admission reads them
      s->waiting.erase(s->waiting.begin());
      insert_by_arrival(s->running, moved);
      ++o.num_admitted;
    }
  }

  // 5. one token for every request that was running before the admissions
  {
    std::vector<int64_t> ids;
    std::vector<int32_t> id_rows, before;
    for (const Req& r : s->running) {
      if (admitted.count(r.seq)) continue;
      ids.push_back(r.seq);
      id_rows.push_back(r.row);
      before.push_back(s->seq_of(r.seq).tokens);
    }
    const size_t n = ids.size();
    std::vector<int64_t> sl(n > 0 ? n : 1), cw(2 * (n > 0 ? n : 1));
    int32_t nc = 0;
    pa_status_t st = pa_bm_append_tokens(bm, ids.data(), int32_t(n), sl.data(), cw.data(), &nc);
    if (st != PA_OK) return st;
    for (size_t i = 0; i < n; ++i) {
      s->slots.push_back(sl[i]);
      s->rows.push_back(id_rows[i]);
      s->positions.push_back(before[i]);
    }
    s->cow.insert(s->cow.end(), cw.begin(), cw.begin() + 2 * nc);
  }

  // 6. lengths per row (0 = empty row)
  for (int32_t r = 0; r < s->max_rows; ++r) {
    const int64_t id = s->row_seq[size_t(r)];
    s->ctx[size_t(r)] = id < 0 ? 0 : s->seq_of(id).tokens;
  }

  o.num_tokens = int32_t(s->slots.size());
  o.slots = s->slots.data();
  o.token_rows = s->rows.data();
  o.token_positions = s->positions.data();
  o.num_rows = s->max_rows;
  o.context_lens = s->ctx.data();
  o.row_seq = s->row_seq.data();
  o.num_swap_out = int32_t(s->swap_out.size() / 2);
  o.swap_out_pairs = s->swap_out.data();
  o.num_swap_in = int32_t(s->swap_in.size() / 2);
  o.swap_in_pairs = s->swap_in.data();
  o.num_cow = int32_t(s->cow.size() / 2);
  o.cow_pairs = s->cow.data();
  o.num_patches = int32_t(s->patches.size() / 3);
  o.table_patches = s->patches.data();
  o.num_finished = int32_t(s->finished.size());
  o.finished = s->finished.data();
  o.num_running = int32_t(s->running.size());
  o.num_waiting = int32_t(s->waiting.size());
  o.num_swapped = int32_t(s->swapped.size());
  s->out = o;
  *out = o;
  return PA_OK;
}

}  // extern "C"
