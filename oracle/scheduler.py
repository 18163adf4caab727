"""Plain Python model of the continuous-batching step scheduler.

Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline use this module; the library never does.

Pages cited (by title and section):
  [OS]  "PagedAttention: How vLLM Serves AI Like an Operating System"
  [VIZ] "vLLM Architecture and PagedAttention - Interactive Visualization"

What it models: requests enter and leave the running batch at every step,
a finished request's place going to a waiting one, and only block tables
change when they do ([OS] "Continuous Batching: The Other Half"; [VIZ]
Continuous Batching); the scheduler checks the free blocks, picks each
step's requests, and preempts low-priority requests by moving their blocks
to CPU memory ([OS] "vLLM Architecture").

Readings where the pages are silent (the same rules the library documents):
  * priority is arrival order; a running request keeps its batch row; a new
    or returning request takes the lowest free row;
  * a step: (1) free requests that reached their final length; (2) reserve
    the blocks each running request's next token needs and, while they do
    not fit, preempt the latest arrival: to the host pool when it has room,
    else free it and requeue it with its tokens so far as its prompt;
    (3) swap requests back in, earliest first, while a row and their blocks
    plus the reserve are free, never one preempted in the same step;
    (4) only with nothing swapped out, admit waiting requests, earliest first,
    while a row and their prompt blocks are free and the step's tokens stay
    within the budget (the first admission is always allowed); (5) every
    request that was running before the admissions appends one token;
  * the step's token list holds the admitted prompts (admission order) and
    then the appended tokens (priority order); swapped-in requests' table
    entries are listed as (row, logical block, physical block) patches;
  * a request submitted with its prompt's token ids (prefix caching on) is
    admitted through the prefix cache: it needs only the blocks it takes
    (fresh ones, and cached ones claimed back from the evictable list), only
    its prompt tokens after the cached ones are written, and its cached
    blocks' table entries are listed as patches; the token
    budget still counts its whole prompt; a request preempted for recompute
    comes back by count, without ids.
"""

from bisect import insort

from .block_manager import BadRequest


class RefScheduler:
    def __init__(self, bm, max_rows: int, max_blocks_per_seq: int, max_batched_tokens: int):
        if max_rows <= 0 or max_blocks_per_seq <= 0 or max_batched_tokens <= 0:
            raise BadRequest("positive sizes")
        self.bm = bm
        self.max_rows = max_rows
        self.max_blocks = max_blocks_per_seq
        self.budget = max_batched_tokens
        self.arrivals = 0
        self.req = {}          # seq -> {"arrival", "prompt", "total", "row"}
        self.waiting = []      # sorted (arrival, seq)
        self.running = []      # sorted (arrival, seq)
        self.swapped = []      # sorted (arrival, seq)
        self.rows = [-1] * max_rows

    def submit(self, seq, prompt_tokens: int, total_tokens: int, prompt_ids=None) -> None:
        if not 1 <= prompt_tokens <= total_tokens or seq < 0:
            raise BadRequest("need 1 <= prompt <= total and a request id >= 0")
        if prompt_ids is not None and (not self.bm.prefix_cache or len(prompt_ids) != prompt_tokens):
            raise BadRequest("token ids need prefix caching on and one id per prompt token")
        if self.bm._nblocks(total_tokens) > min(self.max_blocks, self.bm.num_blocks):
            raise BadRequest("request can never fit")
        if seq in self.req or seq in self.bm.seqs:
            raise BadRequest("duplicate request")
        self.req[seq] = {"arrival": self.arrivals, "prompt": prompt_tokens, "total": total_tokens, "row": -1,
                         "ids": None if prompt_ids is None else [int(t) for t in prompt_ids]}
        self.waiting.append((self.arrivals, seq))
        self.arrivals += 1

    # -- what appending one token to every running request would take --------
    def _need(self) -> int:
        """Blocks one more token for each running request takes (fresh or copy)."""
        need = 0
        refs = {}
        for _, s in self.running:
            st = self.bm.seqs[s]
            if st["n"] % self.bm.bs == 0:
                need += 1
            else:
                last = st["blocks"][-1]
                r = refs.get(last, self.bm.ref[last])
                if r > 1:
                    need += 1
                    refs[last] = r - 1
        return need

    def _free_row(self) -> int:
        return self.rows.index(-1) if -1 in self.rows else -1

    def step(self) -> dict:
        bm = self.bm
        out = {"slots": [], "token_rows": [], "token_positions": [], "swap_out": [], "swap_in": [], "cow": [],
               "patches": [], "finished": [], "num_admitted": 0, "num_swapped_in": 0, "num_preempted_swap": 0,
               "num_preempted_recompute": 0, "num_cached_tokens": 0}

        # 1. retire
        for arrival, s in list(self.running):
            r = self.req[s]
            if bm.num_tokens(s) >= r["total"]:
                bm.free_seq(s)
                self.rows[r["row"]] = -1
                self.running.remove((arrival, s))
                del self.req[s]
                out["finished"].append(s)

        # 2. reserve the next token of every running request; preempt while short
        preempted = set()
        reserve = self._need()
        while reserve > bm.num_free() and self.running:
            arrival, s = self.running.pop()
            r = self.req[s]
            self.rows[r["row"]] = -1
            r["row"] = -1
            preempted.add(s)
            if len(bm.seqs[s]["blocks"]) <= bm.num_free_host():
                out["swap_out"] += bm.swap_out([s])
                insort(self.swapped, (arrival, s))
                out["num_preempted_swap"] += 1
            else:
                r["prompt"] = bm.num_tokens(s)
                r["ids"] = None  # readmitted by count
                bm.free_seq(s)
                insort(self.waiting, (arrival, s))
                out["num_preempted_recompute"] += 1
            reserve = self._need()

        # 3. swap back in
        while self.swapped:
            arrival, s = self.swapped[0]
            if s in preempted:
                break
            row = self._free_row()
            if row < 0:
                break
            n = bm.num_tokens(s)
            grow = 1 if n % bm.bs == 0 else 0
            if len(bm.seqs[s]["blocks"]) + grow + reserve > bm.num_free():
                break
            out["swap_in"] += bm.swap_in([s])
            reserve += grow
            self.req[s]["row"] = row
            self.rows[row] = s
            for j, b in enumerate(bm.seqs[s]["blocks"]):
                out["patches"].append((row, j, b))
            self.swapped.pop(0)
            insort(self.running, (arrival, s))
            out["num_swapped_in"] += 1

        # 4. admit
        admitted = set()
        if not self.swapped:
            left = self.budget - len(self.running)
            while self.waiting:
                arrival, s = self.waiting[0]
                r = self.req[s]
                row = self._free_row()
                if row < 0:
                    break
                take = bm._nblocks(r["prompt"])
                if r["ids"] is not None:  # cached prefix blocks are shared; claiming an evictable one uses it up
                    hits, claimed = bm.prefix_hits(r["ids"])
                    take = take - len(hits) + claimed
                if take + reserve > bm.num_free():
                    break
                if admitted and r["prompt"] > left:
                    break
                first = 0
                if r["ids"] is not None:
                    first = bm.add_seq_tokens(s, r["ids"])
                    out["num_cached_tokens"] += first
                    r["ids"] = None
                else:
                    bm.add_seq(s, r["prompt"])
                blocks = bm.seqs[s]["blocks"]
                for j in range(first // bm.bs):  # cached blocks are not written: their entries are patched
                    out["patches"].append((row, j, blocks[j]))
                for p in range(first, r["prompt"]):
                    out["slots"].append(blocks[p // bm.bs] * bm.bs + p % bm.bs)
                    out["token_rows"].append(row)
                    out["token_positions"].append(p)
                left -= r["prompt"]
                r["row"] = row
                self.rows[row] = s
                admitted.add(s)
                self.waiting.pop(0)
                insort(self.running, (arrival, s))
                out["num_admitted"] += 1

        # 5. one token for every request that ran before the admissions
        grow_seqs = [s for _, s in self.running if s not in admitted]
        before = [bm.num_tokens(s) for s in grow_seqs]
        slots, cows = bm.append_tokens(grow_seqs)
        for s, sl, p in zip(grow_seqs, slots, before):
            out["slots"].append(sl)
            out["token_rows"].append(self.req[s]["row"])
            out["token_positions"].append(p)
        out["cow"] += cows

        out["context_lens"] = [bm.num_tokens(s) if s >= 0 else 0 for s in self.rows]
        out["row_seq"] = list(self.rows)
        out["num_running"] = len(self.running)
        out["num_waiting"] = len(self.waiting)
        out["num_swapped"] = len(self.swapped)
        return out
