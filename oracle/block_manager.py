"""Plain Python model of the KV block manager.

Pages cited (by title and section):
  [OS]  "PagedAttention: How vLLM Serves AI Like an Operating System"
  [VIZ] "vLLM Architecture and PagedAttention - Interactive Visualization"

What it models:
  * one pool of fixed blocks of 16 tokens (32 and 64 as variants); a per-sequence block table maps
    logical block i to a physical block; the free list holds blocks no
    sequence uses ([OS] "PagedAttention: Virtual Memory for KV Cache", How It
    Works and the memory-layout example with its free list);
  * allocation on demand: a sequence gets a new block only when a token lands
    at offset 0 of a fresh block, so a sequence of n tokens holds ceil(n/16)
    blocks and wastes at most 15 slots ([OS] "The Magic: No Pre-allocation");
  * release on finish: a finished sequence gives its blocks back at once
    ([VIZ] Page Table Visualization);
  * sharing with reference counts and copy-on-write: forks for parallel
    sampling share every block, sequences on a common system prompt share its
    blocks, and a shared block is copied before a sequence writes into it
    ([OS] "Copy-on-Write: Sharing KV Cache", Parallel Sampling and Prefix
    Caching).

Readings where the pages are silent:
  * the free list is a queue: allocation takes its head, a block whose
    reference count drops to zero joins its tail; its initial order is an
    input (ascending when none is given);
  * a shared prefix is a whole number of blocks;
  * a write into a block with reference count > 1 first moves the writer onto
    a fresh copy (the pair (old, new) is reported for the device copy) and
    drops one reference from the old block;
  * a freed sequence releases its blocks in logical order;
  * every update is all-or-nothing: when the pool cannot supply the blocks an
    operation needs, it raises NoSpace and leaves the state untouched.

Swap pool ([OS] "vLLM Architecture": a preempted request's blocks move to
CPU memory).  Readings:
  * the host pool is a second set of block ids with its own queue (ascending
    at first) and reference counts;
  * swapping a list of sequences out copies each distinct device block of
    the list once, in list order and logical order; references held by the
    listed sequences move to the host copy, a device block whose count drops
    to zero is released; swapping in is the mirror image into fresh device
    blocks;
  * a swapped-out sequence keeps its length and cannot be appended to,
    forked, used as a prefix or tabled until it is swapped back in; freeing
    it releases its host blocks.
"""

from collections import OrderedDict, deque

BLOCK_SIZE = 16


class NoSpace(Exception):
    """The pool has fewer free blocks than the operation needs."""


class BadRequest(Exception):
    """Unknown / duplicate sequence, or arguments outside the contract."""


class RefBlockManager:
    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE, free_order=None):
        if block_size not in (16, 32, 64):
            raise BadRequest("block_size must be 16, 32 or 64")
        self.bs = int(block_size)
        self.num_blocks = int(num_blocks)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise BadRequest("free_order must be a permutation of the pool")
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.seqs = {}  # seq id -> {"blocks": [...], "n": tokens, "host": bool}
        self.num_host_blocks = 0
        self.host_free = deque()
        self.host_ref = []
        self.prefix_cache = False
        self.cache = {}            # whole prefix (tuple of token ids up to a block's end) -> block
        self.block_key = {}        # block -> its prefix
        self.lru = OrderedDict()   # cached blocks nobody holds; the first is evicted first

    # -- queries ---------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free) + len(self.lru)

    def refcount(self, block: int) -> int:
        return self.ref[block]

    def usage(self) -> float:
        return (self.num_blocks - self.num_free()) / self.num_blocks

    def blocks_of(self, seq):
        return list(self.seqs[seq]["blocks"])

    def num_tokens(self, seq) -> int:
        return self.seqs[seq]["n"]

    # -- helpers -----------------------------------------------------------
    def _take(self) -> int:
        if self.free:
            b = self.free.popleft()
        else:  # evict the cached block released longest ago
            b, _ = self.lru.popitem(last=False)
            del self.cache[self.block_key.pop(b)]
        self.ref[b] = 1
        return b

    def _drop(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.block_key:
                self.lru[b] = None
            else:
                self.free.append(b)

    def _snapshot(self):
        return (deque(self.free), list(self.ref), {k: dict(v, blocks=list(v["blocks"])) for k, v in self.seqs.items()},
                dict(self.cache), dict(self.block_key), OrderedDict(self.lru))

    def _restore(self, saved) -> None:
        self.free, self.ref, self.seqs, self.cache, self.block_key, self.lru = saved

    def _on_host(self, seq) -> bool:
        return bool(self.seqs[seq].get("host"))

    def _take_host(self) -> int:
        h = self.host_free.popleft()
        self.host_ref[h] = 1
        return h

    def _drop_host(self, h: int) -> None:
        self.host_ref[h] -= 1
        if self.host_ref[h] == 0:
            self.host_free.append(h)

    def _nblocks(self, n: int) -> int:
        return -(-n // self.bs)

    # -- updates -----------------------------------------------------------
    def add_seq(self, seq, num_tokens: int) -> None:
        if seq in self.seqs or num_tokens < 0:
            raise BadRequest("duplicate sequence or negative length")
        need = self._nblocks(num_tokens)
        if need > self.num_free():
            raise NoSpace()
        self.seqs[seq] = {"blocks": [self._take() for _ in range(need)], "n": num_tokens}

    def add_seq_with_prefix(self, seq, prefix_seq, prefix_tokens: int, tail_tokens: int) -> None:
        if seq in self.seqs or prefix_seq not in self.seqs or self._on_host(prefix_seq):
            raise BadRequest("duplicate sequence, or unknown or swapped-out prefix sequence")
        if prefix_tokens % self.bs or not 0 <= prefix_tokens <= self.seqs[prefix_seq]["n"] or tail_tokens < 0:
            raise BadRequest("a shared prefix is a whole number of blocks inside the prefix sequence")
        shared = self.seqs[prefix_seq]["blocks"][: prefix_tokens // self.bs]
        need = self._nblocks(tail_tokens)
        if need > self.num_free():
            raise NoSpace()
        for b in shared:
            self.ref[b] += 1
        own = [self._take() for _ in range(need)]
        self.seqs[seq] = {"blocks": list(shared) + own, "n": prefix_tokens + tail_tokens}

    def fork(self, parent, child) -> None:
        if parent not in self.seqs or child in self.seqs or self._on_host(parent):
            raise BadRequest("unknown or swapped-out parent, or duplicate child")
        blocks = list(self.seqs[parent]["blocks"])
        for b in blocks:
            self.ref[b] += 1
        self.seqs[child] = {"blocks": blocks, "n": self.seqs[parent]["n"]}

    def free_seq(self, seq) -> None:
        if seq not in self.seqs:
            raise BadRequest("unknown sequence")
        st = self.seqs.pop(seq)
        if st.get("host"):
            for h in st["blocks"]:
                self._drop_host(h)
        else:
            # with prefix caching the deepest block goes first, so a prefix is evicted from its end
            for b in (reversed(st["blocks"]) if self.prefix_cache else st["blocks"]):
                self._drop(b)

    def append_tokens(self, seqs):
        """Append one token to each listed sequence, in list order.

        Returns (slots, cow_pairs): the slot of every appended token and the
        (src, dst) block copies the device must perform first.  A sequence may
        appear several times (it then receives several consecutive tokens).
        """
        seqs = [s for s in seqs]
        for s in seqs:
            if s not in self.seqs or self._on_host(s):
                raise BadRequest("unknown or swapped-out sequence")
        # all-or-nothing: run the updates on a copy and commit on success
        saved = self._snapshot()
        try:
            slots, cows = [], []
            for s in seqs:
                st = self.seqs[s]
                pos = st["n"]
                if pos % self.bs == 0:
                    if not self.num_free():
                        raise NoSpace()
                    st["blocks"].append(self._take())
                else:
                    last = st["blocks"][-1]
                    if self.ref[last] > 1:
                        if not self.num_free():
                            raise NoSpace()
                        fresh = self._take()
                        self.ref[last] -= 1
                        st["blocks"][-1] = fresh
                        cows.append((last, fresh))
                slots.append(st["blocks"][pos // self.bs] * self.bs + pos % self.bs)
                st["n"] = pos + 1
            return slots, cows
        except NoSpace:
            self._restore(saved)
            raise

    # -- prefix cache ------------------------------------------------------
    def enable_prefix_cache(self) -> None:
        if self.prefix_cache or self.seqs:
            raise BadRequest("turn prefix caching on once, before the first sequence")
        self.prefix_cache = True

    def num_cached_free(self) -> int:
        return len(self.lru)

    def prefix_hits(self, tokens):
        """The cached blocks of the longest cached prefix of ``tokens``, and how
        many of them wait in the evictable list.  Changes nothing."""
        tokens = [int(t) for t in tokens]
        hits = []
        for i in range(len(tokens) // self.bs):
            b = self.cache.get(tuple(tokens[: self.bs * (i + 1)]))
            if b is None:
                break
            hits.append(b)
        return hits, sum(1 for b in hits if b in self.lru)

    def add_seq_tokens(self, seq, tokens) -> int:
        """New sequence from its token ids, sharing the cached blocks of its
        longest cached prefix; returns how many leading tokens were cached."""
        if not self.prefix_cache:
            raise BadRequest("prefix caching is off")
        if seq in self.seqs:
            raise BadRequest("duplicate sequence")
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        full, total = n // self.bs, self._nblocks(n)
        prefixes = [tuple(tokens[: self.bs * (i + 1)]) for i in range(full)]
        hits = []
        for p in prefixes:
            if p not in self.cache:
                break
            hits.append(self.cache[p])
        claimed = sum(1 for b in hits if b in self.lru)
        if total - len(hits) > self.num_free() - claimed:
            raise NoSpace()
        for b in hits:
            self.lru.pop(b, None)
            self.ref[b] += 1
        blocks = list(hits)
        for i in range(len(hits), total):
            b = self._take()
            blocks.append(b)
            if i < full:
                old = self.cache.get(prefixes[i])
                if old is not None:  # an evictable block held this prefix: the new one takes it over
                    del self.block_key[old]
                    if old in self.lru:
                        del self.lru[old]
                        self.free.append(old)
                self.cache[prefixes[i]] = b
                self.block_key[b] = prefixes[i]
        self.seqs[seq] = {"blocks": blocks, "n": n}
        return len(hits) * self.bs

    # -- swap pool ---------------------------------------------------------
    def set_host_pool(self, num_host_blocks: int) -> None:
        if self.num_host_blocks or num_host_blocks < 0:
            raise BadRequest("the host pool is set once, with a size >= 0")
        self.num_host_blocks = int(num_host_blocks)
        self.host_free = deque(range(num_host_blocks))
        self.host_ref = [0] * num_host_blocks

    def is_swapped(self, seq) -> bool:
        return self._on_host(seq)

    def num_free_host(self) -> int:
        return len(self.host_free)

    def host_refcount(self, block: int) -> int:
        return self.host_ref[block]

    def _check_swap_list(self, seqs, want_host: bool):
        if len(set(seqs)) != len(seqs):
            raise BadRequest("a sequence is listed twice")
        for s in seqs:
            if s not in self.seqs or self._on_host(s) != want_host:
                raise BadRequest("unknown sequence or wrong residence")

    def swap_out(self, seqs):
        """Move the listed sequences' blocks to the host pool.

        Returns the (device block, host block) copies, one per distinct device
        block, in list order and logical order.
        """
        seqs = list(seqs)
        self._check_swap_list(seqs, False)
        distinct = {b for s in seqs for b in self.seqs[s]["blocks"]}
        if len(distinct) > len(self.host_free):
            raise NoSpace()
        where, pairs = {}, []
        for s in seqs:
            st = self.seqs[s]
            moved = []
            for b in st["blocks"]:
                if b in where:
                    self.host_ref[where[b]] += 1
                else:
                    where[b] = self._take_host()
                    pairs.append((b, where[b]))
                self._drop(b)
                moved.append(where[b])
            st["blocks"], st["host"] = moved, True
        return pairs

    def swap_in(self, seqs):
        """Bring swapped-out sequences back into fresh device blocks.

        Returns the (host block, device block) copies, one per distinct host
        block, in list order and logical order.
        """
        seqs = list(seqs)
        self._check_swap_list(seqs, True)
        distinct = {h for s in seqs for h in self.seqs[s]["blocks"]}
        if len(distinct) > self.num_free():
            raise NoSpace()
        where, pairs = {}, []
        for s in seqs:
            st = self.seqs[s]
            moved = []
            for h in st["blocks"]:
                if h in where:
                    self.ref[where[h]] += 1
                else:
                    where[h] = self._take()
                    pairs.append((h, where[h]))
                self._drop_host(h)
                moved.append(where[h])
            st["blocks"], st["host"] = moved, False
        return pairs

    def append_token(self, seq):
        slots, cows = self.append_tokens([seq])
        return slots[0], (cows[0] if cows else (-1, -1))

    def block_table(self, seqs, max_blocks: int, pad: int = -1):
        """Rows of logical -> physical ids (padded with ``pad``) and context lengths."""
        table, ctx = [], []
        for s in seqs:
            if s not in self.seqs or self._on_host(s):
                raise BadRequest("unknown or swapped-out sequence")
            blocks = self.seqs[s]["blocks"]
            if len(blocks) > max_blocks:
                raise BadRequest("table too narrow")
            table.append(list(blocks) + [pad] * (max_blocks - len(blocks)))
            ctx.append(self.seqs[s]["n"])
        return table, ctx
