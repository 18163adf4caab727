"""Pins of the oracle block manager against the pages' worked examples.

Each test reproduces an example the pages print (fixtures under
tests/golden/, each naming its page and section) or a bound they state.
"""
import numpy as np
import pytest

from oracle.block_manager import BadRequest, NoSpace, RefBlockManager
from tests._golden import load


def physical_map(bm, names):
    """Render the pool as the memory-layout example does: [Seq:logical] or [free]."""
    cells = ["[free]"] * bm.num_blocks
    for name in names:
        for j, b in enumerate(bm.blocks_of(name)):
            cells[b] = f"[{name}:{j}]"
    return "".join(cells)


def test_worked_memory_layout_example():
    g = load("os_memory_layout.txt")
    bm = RefBlockManager(g["num_blocks"], free_order=g["free_order"])
    for name in ("A", "B", "C"):
        bm.add_seq(name, g["lengths"][name])
    assert bm.blocks_of("A") == g["table_A"]
    assert bm.blocks_of("B") == g["table_B"]
    assert bm.blocks_of("C") == g["table_C"]
    assert list(bm.free) == g["free_after"]
    assert physical_map(bm, ["A", "B", "C"]) == g["physical_map"]
    table, ctx = bm.block_table(["A", "B", "C"], 3, pad=-1)
    assert table == [[0, 2, 6], [4, 7, 1], [3, 9, -1]]
    assert ctx == [40, 48, 17]


@pytest.mark.parametrize("lens", [(33, 33, 17), (48, 48, 32), (40, 35, 20)])
def test_worked_example_any_lengths_in_range(lens):
    g = load("os_memory_layout.txt")
    bm = RefBlockManager(g["num_blocks"], free_order=g["free_order"])
    for name, n in zip("ABC", lens):
        bm.add_seq(name, n)
    assert physical_map(bm, ["A", "B", "C"]) == g["physical_map"]


def test_on_demand_allocation_schedule():
    g = load("os_no_prealloc.txt")
    bm = RefBlockManager(200)
    bm.add_seq("A", 0)
    alloc_at = []
    for token in range(1, g["tokens"] + 1):
        before = len(bm.blocks_of("A"))
        bm.append_token("A")
        if len(bm.blocks_of("A")) > before:
            alloc_at.append(token)
    assert alloc_at[:3] == g["first_alloc_tokens"]
    assert alloc_at == list(range(1, g["tokens"] + 1, 16))
    assert len(bm.blocks_of("A")) == g["blocks_at_end"]


@pytest.mark.parametrize("n", list(range(0, 70)) + [1199, 1200, 1201, 8191, 8192])
def test_internal_waste_bound(n):
    g = load("os_no_prealloc.txt")
    bm = RefBlockManager(1024)
    bm.add_seq("s", n)
    nb = len(bm.blocks_of("s"))
    assert nb == -(-n // 16)
    waste = nb * 16 - n
    assert 0 <= waste <= g["max_waste_slots"]


def test_parallel_sampling_example():
    g = load("os_parallel_sampling.txt")
    bm = RefBlockManager(32)
    bm.add_seq("prompt", 96)
    assert bm.blocks_of("prompt") == g["prompt_blocks"]
    outs = [f"out{i}" for i in range(g["n"])]
    for o in outs:
        bm.fork("prompt", o)
    bm.free_seq("prompt")
    for o in outs:
        for _ in range(32):
            bm.append_token(o)
    for o, uniq in zip(outs, g["unique_blocks"]):
        assert bm.blocks_of(o) == g["prompt_blocks"] + uniq
    for b in g["prompt_blocks"]:
        assert bm.refcount(b) == g["n"]
    shared_prompt_blocks = {b for o in outs for b in bm.blocks_of(o)[:6]}
    assert len(shared_prompt_blocks) == g["prompt_blocks_shared"]
    assert g["n"] * len(g["prompt_blocks"]) == g["prompt_blocks_unshared"]
    assert bm.num_free() == 32 - 14


def test_prefix_caching_example():
    g = load("os_prefix_caching.txt")
    bm = RefBlockManager(64)
    bm.add_seq("sys", 64)
    assert bm.blocks_of("sys") == g["system_blocks"]
    tails = [48, 40, 32]  # 3, 3 and 2 blocks
    for i, (tail, uniq) in enumerate(zip(tails, g["request_unique"])):
        bm.add_seq_with_prefix(f"r{i}", "sys", 64, tail)
        assert bm.blocks_of(f"r{i}") == g["system_blocks"] + uniq


def test_prefix_caching_thousand_users():
    g = load("os_prefix_caching.txt")
    bm = RefBlockManager(4 + g["users"])
    bm.add_seq("sys", 64)
    for u in range(g["users"]):
        bm.add_seq_with_prefix(u, "sys", 64, 10)
    system = {b for u in range(g["users"]) for b in bm.blocks_of(u)[:4]}
    assert len(system) == g["system_blocks_shared"]
    assert g["users"] * 4 == g["system_blocks_unshared"]
    for b in g["system_blocks"]:
        assert bm.refcount(b) == g["users"] + 1
    assert bm.num_free() == 0


def test_page_table_release_on_finish():
    g = load("viz_page_table.txt")
    bm = RefBlockManager(g["pool_pages"], free_order=np.random.default_rng(0).permutation(g["pool_pages"]))
    bm.add_seq(0, g["seq0_pages"] * g["page_tokens"] - 5)
    for s in range(1, g["sequences"]):
        bm.add_seq(s, 20 + 7 * s)
    assert len(bm.blocks_of(0)) == g["seq0_pages"]
    before = bm.num_free()
    bm.free_seq(0)
    assert bm.num_free() == before + g["seq0_pages"]
    assert bm.usage() == pytest.approx((g["pool_pages"] - bm.num_free()) / g["pool_pages"])


def test_copy_on_write_for_a_shared_partial_block():
    bm = RefBlockManager(16)
    bm.add_seq("p", 90)  # 6 blocks, the last holds 10 of 16 tokens
    kids = ["c0", "c1", "c2", "c3"]
    for c in kids:
        bm.fork("p", c)
    bm.free_seq("p")
    last = bm.blocks_of("c0")[-1]
    assert bm.refcount(last) == 4
    pairs = []
    for c in kids:
        slot, cow = bm.append_token(c)
        pairs.append(cow)
        assert slot == bm.blocks_of(c)[-1] * 16 + 10
    # the first three writers move to copies; the last one owns the original
    assert [p[0] for p in pairs[:3]] == [last] * 3
    assert len({p[1] for p in pairs[:3]}) == 3
    assert pairs[3] == (-1, -1)
    assert bm.blocks_of("c3")[-1] == last
    assert bm.refcount(last) == 1
    for b in bm.blocks_of("c0")[:-1]:
        assert bm.refcount(b) == 4


def test_no_space_is_all_or_nothing():
    bm = RefBlockManager(4)
    bm.add_seq("a", 40)  # 3 blocks
    snapshot = (list(bm.free), list(bm.ref), {k: dict(v, blocks=list(v["blocks"])) for k, v in bm.seqs.items()})
    with pytest.raises(NoSpace):
        bm.add_seq("b", 20)  # needs 2
    with pytest.raises(NoSpace):
        bm.append_tokens(["a"] * 8 + ["a"] * 20)  # crosses two block boundaries
    assert (list(bm.free), list(bm.ref)) == snapshot[:2]
    assert bm.blocks_of("a") == snapshot[2]["a"]["blocks"] and bm.num_tokens("a") == 40
    with pytest.raises(BadRequest):
        bm.add_seq("a", 1)
    with pytest.raises(BadRequest):
        bm.add_seq_with_prefix("c", "a", 10, 0)  # not a whole block


def test_freed_blocks_join_the_tail_of_the_free_list():
    bm = RefBlockManager(6)
    bm.add_seq("a", 32)  # blocks 0, 1
    bm.add_seq("b", 16)  # block 2
    bm.free_seq("a")
    assert list(bm.free) == [3, 4, 5, 0, 1]
    bm.add_seq("c", 48)
    assert bm.blocks_of("c") == [3, 4, 5]
