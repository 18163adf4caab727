"""Planted mistakes in the oracle must each break at least one pin.

Each case takes the source of one oracle function, changes one expression
into a plausible mistake (a dropped term, a wrong index, an off-by-one), runs
the changed function in place of the real one, and checks that the named pin
then fails.  Everything here runs on the CPU against the oracle only.
"""
import inspect
import textwrap

import pytest

import oracle.attention
import oracle.block_manager
import oracle.layout
import oracle.scheduler
from tests import test_oracle_attention as PA
from tests import test_oracle_block_manager as PB
from tests import test_prefix_cache as PC
from tests import test_scheduler as PS

MUTATIONS = [
    # (module, function or Class.method, original text, planted mistake, pin, pin args)
    (oracle.attention, "decode", "g = h // G", "g = h % Hkv",
     PA.test_query_heads_read_their_contiguous_kv_group, ()),
    (oracle.attention, "decode", "z = scale * (K[g] @ qf[s, h])", "z = K[g] @ qf[s, h]",
     PA.test_decode_matches_brute_force_on_the_tiny_shape, ("f32", 16)),
    (oracle.attention, "decode", "out[s, h] = _softmax_weighted_sum(z, V[g])",
     "out[s, h] = _softmax_weighted_sum(z, K[g])",
     PA.test_decode_matches_brute_force_on_the_tiny_shape, ("bf16", 16)),
    (oracle.attention, "prefill_chunk", "last = n - C + i", "last = n - C + i - 1",
     PA.test_prefill_matches_brute_force, (16,)),
    (oracle.attention, "prefill_chunk", "last = n - C + i", "last = n - 1",
     PA.test_chunk_of_one_is_decode_and_rows_are_causal, ()),
    (oracle.attention, "gather_kv", "K = K.transpose(1, 0, 2, 3)", "K = K.transpose(0, 1, 2, 3)",
     PA.test_decode_matches_brute_force_on_the_tiny_shape, ("f16", 16)),
    (oracle.attention, "gather_kv", "phys = np.asarray(table_row[:nb], dtype=np.int64)",
     "phys = np.arange(nb, dtype=np.int64)",
     PA.test_decode_matches_brute_force_on_the_tiny_shape, ("f32", 16)),
    (oracle.attention, "gather_kv", "V = V.transpose(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :ctx]",
     "V = V.transpose(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :nb * bs][:, :ctx + 1]",
     PA.test_unread_table_entries_and_tail_slots_do_not_matter, ()),
    (oracle.attention, "to_f64", "<< np.uint32(16)", "<< np.uint32(15)",
     PA.test_bf16_bit_patterns_decode_exactly, ()),
    (oracle.attention, "reshape_and_cache", "b, o = divmod(slot, bs)", "o, b = divmod(slot, bs)",
     PA.test_cache_write_lands_at_the_layout_offsets, ()),
    (oracle.layout, "k_offset", "((d // 8) * 16 + t) * 8 + d % 8", "(t * 16 + d // 8) * 8 + d % 8",
     PA.test_tile_layout_matches_hand_derived_offsets, ()),
    (oracle.layout, "v_offset", "((d // 16) % 2) * 4 + t % 4", "((d // 16) % 2) + (t % 4) * 2",
     PA.test_tile_layout_matches_hand_derived_offsets, ()),
    (oracle.block_manager, "RefBlockManager.append_tokens", "if pos % self.bs == 0:",
     "if pos % self.bs == 1 or pos == 0:",
     PB.test_on_demand_allocation_schedule, ()),
    (oracle.block_manager, "RefBlockManager.append_tokens", "self.ref[last] -= 1", "pass",
     PB.test_copy_on_write_for_a_shared_partial_block, ()),
    (oracle.block_manager, "RefBlockManager.append_tokens", "if self.ref[last] > 1:", "if False:",
     PB.test_copy_on_write_for_a_shared_partial_block, ()),
    (oracle.block_manager, "RefBlockManager._drop", "self.free.append(b)", "self.free.appendleft(b)",
     PB.test_freed_blocks_join_the_tail_of_the_free_list, ()),
    (oracle.block_manager, "RefBlockManager.fork", "self.ref[b] += 1", "pass",
     PB.test_parallel_sampling_example, ()),
    (oracle.block_manager, "RefBlockManager.add_seq_with_prefix",
     "shared = self.seqs[prefix_seq][\"blocks\"][: prefix_tokens // self.bs]",
     "shared = self.seqs[prefix_seq][\"blocks\"][: prefix_tokens // self.bs - 1]",
     PB.test_prefix_caching_example, ()),
    (oracle.layout, "block_index", "(t // BLOCK_SIZE) * BLOCK_SIZE * head_dim", "(t // BLOCK_SIZE) * head_dim",
     PA.test_larger_blocks_are_runs_of_tiles_at_hand_derived_offsets, ()),
    (oracle.attention, "gather_kv", "nb = -(-ctx // bs)", "nb = -(-ctx // 16)",
     PA.test_block_size_changes_nothing_in_the_result, (32,)),
    (oracle.scheduler, "RefScheduler.step", "arrival, s = self.running.pop()", "arrival, s = self.running.pop(0)",
     PS.test_hand_worked_swap_trace, ("oracle",)),
    (oracle.scheduler, "RefScheduler.step", "if bm.num_tokens(s) >= r[\"total\"]:",
     "if bm.num_tokens(s) > r[\"total\"]:", PS.test_oracle_replay_reads_back_every_token, (PS.CASES[0],)),
    (oracle.scheduler, "RefScheduler.step", "out[\"patches\"].append((row, j, b))",
     "out[\"patches\"].append((row, j + 1, b))", PS.test_oracle_replay_reads_back_every_token, (PS.CASES[0],)),
    (oracle.scheduler, "RefScheduler.step", "if not self.swapped:", "if True:",
     PS.test_oracle_replay_reads_back_every_token, (PS.CASES[0],)),
    (oracle.scheduler, "RefScheduler.step", "grow = 1 if n % bm.bs == 0 else 0", "grow = 0",
     PS.test_oracle_replay_reads_back_every_token, (PS.CASES[4],)),
    (oracle.scheduler, "RefScheduler._need", "if st[\"n\"] % self.bm.bs == 0:", "if st[\"n\"] % self.bm.bs == 1:",
     PS.test_oracle_replay_reads_back_every_token, (PS.CASES[0],)),
    (oracle.block_manager, "RefBlockManager.swap_out", "pairs.append((b, where[b]))",
     "pairs.append((where[b], b))", PS.test_oracle_replay_reads_back_every_token, (PS.CASES[0],)),
    (oracle.block_manager, "RefBlockManager.swap_in", "self._drop_host(h)", "pass",
     PS.test_oracle_replay_reads_back_every_token, (PS.CASES[0],)),
    (oracle.block_manager, "RefBlockManager.swap_out", "self.host_ref[where[b]] += 1", "pass",
     PS.test_swap_round_trip_with_shared_blocks_matches_the_oracle, ()),
    (oracle.scheduler, "RefScheduler.step", "out[\"patches\"].append((row, j, blocks[j]))", "pass",
     PS.test_prefix_cached_admission_reads_back_every_token, (PS.PREFIX_CASES[0],)),
    (oracle.scheduler, "RefScheduler.step", "take = take - len(hits) + claimed", "take = take - len(hits)",
     PS.test_prefix_cached_admission_reads_back_every_token, (PS.PREFIX_CASES[1],)),
    (oracle.block_manager, "RefBlockManager._drop", "self.lru[b] = None", "self.free.append(b)",
     PC.test_released_prefixes_wait_in_lru_and_are_evicted_from_their_end, ("oracle",)),
    (oracle.block_manager, "RefBlockManager.free_seq", "reversed(st[\"blocks\"]) if self.prefix_cache",
     "st[\"blocks\"] if self.prefix_cache", PC.test_released_prefixes_wait_in_lru_and_are_evicted_from_their_end,
     ("oracle",)),
    (oracle.block_manager, "RefBlockManager.add_seq_tokens", "tuple(tokens[: self.bs * (i + 1)])",
     "tuple(tokens[self.bs * i: self.bs * (i + 1)])", PC.test_a_block_is_shared_only_under_the_same_prefix,
     ("oracle",)),
    (oracle.block_manager, "RefBlockManager.add_seq_tokens", "if i < full:", "if i <= full:",
     PC.test_only_full_blocks_are_cached_and_a_miss_ends_the_run, ("oracle",)),
    (oracle.attention, "copy_blocks", "k_cache[dst] = k_cache[src]", "k_cache[src] = k_cache[dst]",
     PA.test_copy_blocks_by_hand, ()),
    (oracle.attention, "copy_blocks", "v_cache[dst] = v_cache[src]", "pass",
     PA.test_copy_blocks_by_hand, ()),
    (oracle.attention, "copy_blocks", "k_cache[dst] = k_cache[src]", "pass",
     PA.test_copy_blocks_by_hand, ()),
    (oracle.attention, "copy_blocks", "k_cache[dst] = k_cache[src]", "k_cache[dst, 0] = k_cache[src, 0]",
     PA.test_copy_blocks_by_hand, ()),
    (oracle.attention, "swap_blocks", "dst_k[dst] = src_k[src]", "dst_k[src] = src_k[dst]",
     PA.test_swap_blocks_by_hand, ()),
    (oracle.attention, "swap_blocks", "dst_v[dst] = src_v[src]", "pass",
     PA.test_swap_blocks_by_hand, ()),
    (oracle.attention, "swap_blocks", "dst_k[dst] = src_k[src]", "pass",
     PA.test_swap_blocks_by_hand, ()),
    (oracle.attention, "swap_blocks", "for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):",
     "for dst, src in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):",
     PA.test_swap_blocks_by_hand, ()),
    (oracle.block_manager, "RefBlockManager._take", "b, _ = self.lru.popitem(last=False)",
     "b, _ = self.lru.popitem(last=True)", PC.test_released_prefixes_wait_in_lru_and_are_evicted_from_their_end,
     ("oracle",)),
]


def _mutated(module, qualname, old, new):
    owner = module
    parts = qualname.split(".")
    for p in parts[:-1]:
        owner = getattr(owner, p)
    fn = getattr(owner, parts[-1])
    src = textwrap.dedent(inspect.getsource(fn))
    assert src.count(old) >= 1, f"{qualname}: text to mutate not found"
    src = src.replace(old, new)
    ns = dict(vars(module))
    exec(compile(src, f"<mutant {qualname}>", "exec"), ns)
    return owner, parts[-1], ns[parts[-1]]


@pytest.mark.parametrize("case", range(len(MUTATIONS)),
                         ids=[f"{m[1]}:{m[3][:30]}" for m in MUTATIONS])
def test_planted_mistake_breaks_a_pin(case, monkeypatch):
    module, qualname, old, new, pin, args = MUTATIONS[case]
    pin(*args)  # the pin holds for the real oracle
    owner, name, fn = _mutated(module, qualname, old, new)
    monkeypatch.setattr(owner, name, fn)
    if module is oracle.layout:
        # tile_index reads the offset functions from its module namespace
        monkeypatch.setattr(oracle.layout, name, fn)
    with pytest.raises(Exception):
        pin(*args)
