"""Pins of the attention oracle: brute force, closed forms, the tile layout
definition, paging invariance and the causal chunk placement.

None of these re-types the oracle's formulas: expected values come from the
pure-Python triple loop on logical (unpaged) K/V, from closed forms, from the
hand-derived layout fixture, or from properties the pages fix (paging changes
where values sit, not what attention returns: "PagedAttention: How vLLM Serves
AI Like an Operating System", section "Throughput Impact: The Numbers").
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import attention as A
from oracle import layout as L
from oracle.block_manager import RefBlockManager
from tests._golden import load
from tests.brute import attend
from workloads import make_workload, run_program, to_storage


# ---------------------------------------------------------------- helpers

def paged_from_logical(logical_k, logical_v, num_blocks, dtype, free_order=None, fill=0.0, block_size=16):
    """Place per-sequence logical K/V ([n, Hkv, D] storage arrays) into a pool.

    The block manager hands out slots token by token; the oracle's cache write
    stores each token.  Returns pools, tables and context lengths.
    """
    Hkv, D = logical_k[0].shape[1:]
    sd = logical_k[0].dtype
    k_pool = np.full((num_blocks, Hkv, block_size * D), fill, dtype=sd)
    v_pool = np.full((num_blocks, Hkv, block_size * D), fill, dtype=sd)
    bm = RefBlockManager(num_blocks, block_size=block_size, free_order=free_order)
    for s in range(len(logical_k)):
        bm.add_seq(s, 0)
    # interleave sequences token by token so their blocks interleave in the pool
    longest = max(len(k) for k in logical_k)
    for t in range(longest):
        seqs = [s for s in range(len(logical_k)) if t < len(logical_k[s])]
        slots, cows = bm.append_tokens(seqs)
        assert not cows
        key = np.stack([logical_k[s][t] for s in seqs])
        val = np.stack([logical_v[s][t] for s in seqs])
        A.reshape_and_cache(k_pool, v_pool, key, val, np.array(slots))
    maxb = max(1, max(-(-len(k) // block_size) for k in logical_k))
    table, ctx = bm.block_table(range(len(logical_k)), maxb, pad=-1)
    return k_pool, v_pool, np.array(table, dtype=np.int32), np.array(ctx, dtype=np.int32), bm


def brute_decode(q, logical_k, logical_v, scale, dtype):
    S, Hq, D = q.shape
    Hkv = logical_k[0].shape[1]
    G = Hq // Hkv
    out = np.zeros((S, Hq, D))
    for s in range(S):
        K = A.to_f64(logical_k[s], dtype)
        V = A.to_f64(logical_v[s], dtype)
        qs = A.to_f64(q[s], dtype)
        for h in range(Hq):
            g = h // G
            out[s, h] = attend(list(qs[h]), [list(K[t, g]) for t in range(len(K))],
                               [list(V[t, g]) for t in range(len(V))], scale)
    return out


def random_logical(rng, lens, Hkv, D, dtype):
    ks = [to_storage(rng.standard_normal((n, Hkv, D), dtype=np.float32), dtype) for n in lens]
    vs = [to_storage(rng.standard_normal((n, Hkv, D), dtype=np.float32), dtype) for n in lens]
    return ks, vs


# ---------------------------------------------------------------- layout

def test_tile_layout_matches_hand_derived_offsets():
    g = load("tile_layout.txt")
    for t, d, ko, vo in g["entries"]:
        assert L.k_offset(t, d) == ko, (t, d)
        assert L.v_offset(t, d) == vo, (t, d)


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_tile_layout_is_a_bijection(D):
    for which in ("k", "v"):
        idx = L.tile_index(which, D)
        assert sorted(idx.ravel().tolist()) == list(range(16 * D))


def test_larger_blocks_are_runs_of_tiles_at_hand_derived_offsets():
    """A 32- or 64-token block is 2 or 4 consecutive 16-token tiles, in token order."""
    D = 64
    k32, v32 = L.block_index("k", D, 32), L.block_index("v", D, 32)
    assert k32[17, 5] == 1024 + 13            # tile 1, K(t=1, d=5) = (0 * 16 + 1) * 8 + 5
    assert v32[20, 40] == 1024 + 704          # tile 1, V(t=4, d=40) = ((1 * 4 + 1) * 16 + 8) * 8 + 0 + 0
    assert k32[3, 9] == L.k_offset(3, 9)      # tile 0 is the 16-token tile itself
    k64 = L.block_index("k", D, 64)
    assert k64[63, 63] == 3 * 1024 + L.k_offset(15, 63)
    for bs in (32, 64):
        for which in ("k", "v"):
            idx = L.block_index(which, D, bs)
            assert sorted(idx.ravel().tolist()) == list(range(bs * D))


@pytest.mark.parametrize("bs", [32, 64])
def test_block_size_changes_nothing_in_the_result(bs):
    """The same logical K/V paged in 16-token and larger blocks attend identically."""
    rng = np.random.default_rng(19)
    lens = [70, 5, 129, 33]
    ks, vs = random_logical(rng, lens, 2, 64, "bf16")
    q = to_storage(rng.standard_normal((4, 8, 64), dtype=np.float32), "bf16")
    a = paged_from_logical(ks, vs, 30, "bf16", rng.permutation(30))
    b = paged_from_logical(ks, vs, 30, "bf16", rng.permutation(30), block_size=bs)
    for s, n in enumerate(lens):
        Ka, Va = A.gather_kv(a[0], a[1], a[2][s], n, "bf16")
        Kb, Vb = A.gather_kv(b[0], b[1], b[2][s], n, "bf16", bs)
        assert np.array_equal(Ka, Kb) and np.array_equal(Va, Vb)
    # equal inputs; only the fp64 summation order of the library matmul may differ with the array strides
    np.testing.assert_allclose(A.decode(q, *a[:4], 0.125, "bf16"), A.decode(q, *b[:4], 0.125, "bf16"),
                               rtol=0, atol=1e-12)


def test_cache_write_lands_at_the_layout_offsets():
    D, Hkv = 64, 2
    k = np.zeros((3, Hkv, 16 * D), np.float32)
    v = np.zeros((3, Hkv, 16 * D), np.float32)
    key = np.arange(Hkv * D, dtype=np.float32).reshape(1, Hkv, D) + 1
    val = -key
    A.reshape_and_cache(k, v, key, val, np.array([2 * 16 + 5]))
    # token offset 5 of block 2; dim 17 of head 1 -> K at 297, V at 141 (hand-derived)
    assert k[2, 1, 297] == key[0, 1, 17]
    assert v[2, 1, 141] == val[0, 1, 17]
    assert np.count_nonzero(k) == Hkv * D and np.count_nonzero(v) == Hkv * D
    assert not k[:2].any() and not v[:2].any()


def test_negative_slot_is_skipped():
    k = np.zeros((2, 1, 16 * 32), np.float32)
    v = np.zeros_like(k)
    key = np.ones((2, 1, 32), np.float32)
    A.reshape_and_cache(k, v, key, key, np.array([-1, 17]))
    assert np.count_nonzero(k[0]) == 0 and np.count_nonzero(k[1]) == 32


# ---------------------------------------------------------------- dtype handling

def test_bf16_bit_patterns_decode_exactly():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x3F81, 0x0001], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, math.inf, 1.0 + 2 ** -7, 2.0 ** -133]
    got = A.to_f64(bits, "bf16")
    for g_, w in zip(got, want):
        assert g_ == w


def test_input_rounding_is_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -(1.0 + 2 ** -8)], np.float32)
    got = A.to_f64(to_storage(x, "bf16"), "bf16")
    assert list(got) == [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -1.0]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_output_rounding_to_storage_is_nearest(dtype):
    rng = np.random.default_rng(3)
    a = rng.standard_normal(20000) * 3
    r = A.to_f64(A.round_f64_to(a, dtype), dtype)
    # no representable value lies strictly closer: compare with neighbours
    if dtype == "bf16":
        bits = A.round_f64_to(a, dtype).astype(np.int64)
        up = A.to_f64((bits + 1).astype(np.uint16), dtype)
        dn = A.to_f64((bits - 1).astype(np.uint16), dtype)
    else:
        bits = A.round_f64_to(a, dtype).view(np.uint16).astype(np.int64)
        up = (bits + 1).astype(np.uint16).view(np.float16).astype(np.float64)
        dn = (bits - 1).astype(np.uint16).view(np.float16).astype(np.float64)
    err = np.abs(r - a)
    assert np.all(err <= np.abs(up - a)) and np.all(err <= np.abs(dn - a))


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("dtype,bs", [("f32", 16), ("f16", 16), ("bf16", 16), ("f32", 32), ("bf16", 64)])
def test_decode_matches_brute_force_on_the_tiny_shape(dtype, bs):
    rng = np.random.default_rng(11)
    lens = [20, 37, 16, 1]
    ks, vs = random_logical(rng, lens, 4, 64, dtype)
    q = to_storage(rng.standard_normal((4, 4, 64), dtype=np.float32), dtype)
    k_pool, v_pool, table, ctx, _ = paged_from_logical(ks, vs, 20, dtype, rng.permutation(20), block_size=bs)
    got = A.decode(q, k_pool, v_pool, table, ctx, 1 / 8, dtype)
    want = brute_decode(q, ks, vs, 1 / 8, dtype)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@settings(max_examples=25, deadline=None)
@given(S=st.integers(1, 4), G=st.sampled_from([1, 2, 4]), Hkv=st.integers(1, 2), D=st.sampled_from([32, 64]),
       lens=st.lists(st.integers(1, 40), min_size=4, max_size=4), seed=st.integers(0, 2 ** 31 - 1),
       bs=st.sampled_from([16, 32, 64]))
def test_decode_matches_brute_force_hypothesis(S, G, Hkv, D, lens, seed, bs):
    rng = np.random.default_rng(seed)
    lens = lens[:S]
    ks, vs = random_logical(rng, lens, Hkv, D, "f32")
    q = rng.standard_normal((S, G * Hkv, D)).astype(np.float32)
    nb = sum(-(-n // bs) for n in lens) + 3
    k_pool, v_pool, table, ctx, _ = paged_from_logical(ks, vs, nb, "f32", rng.permutation(nb), fill=np.nan,
                                                        block_size=bs)
    scale = 1 / math.sqrt(D)
    got = A.decode(q, k_pool, v_pool, table, ctx, scale, "f32")
    want = brute_decode(q, ks, vs, scale, "f32")
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("bs", [16, 32])
def test_prefill_matches_brute_force(bs):
    rng = np.random.default_rng(5)
    lens, C, Hkv, G, D = [40, 23], 7, 2, 2, 32
    ks, vs = random_logical(rng, lens, Hkv, D, "bf16")
    k_pool, v_pool, table, ctx, _ = paged_from_logical(ks, vs, 10, "bf16", rng.permutation(10), fill=0,
                                                        block_size=bs)
    q = to_storage(rng.standard_normal((2, C, Hkv * G, D), dtype=np.float32), "bf16")
    got = A.prefill_chunk(q, k_pool, v_pool, table, ctx, 0.25, "bf16")
    for s, n in enumerate(lens):
        for i in range(C):
            last = n - C + i
            want = brute_decode(q[s:s + 1, i], [ks[s][:last + 1]], [vs[s][:last + 1]], 0.25, "bf16")
            np.testing.assert_allclose(got[s, i], want[0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms

def tiny_pool(rng, n, Hkv=1, D=32, dtype="f32"):
    ks, vs = random_logical(rng, [n], Hkv, D, dtype)
    k_pool, v_pool, table, ctx, _ = paged_from_logical(ks, vs, -(-n // 16) + 2, dtype,
                                                        rng.permutation(-(-n // 16) + 2), fill=np.nan)
    return ks[0], vs[0], k_pool, v_pool, table, ctx


def test_single_token_context_returns_its_value_exactly():
    rng = np.random.default_rng(1)
    k, v, kp, vp, table, ctx = tiny_pool(rng, 1, Hkv=2)
    q = rng.standard_normal((1, 4, 32)).astype(np.float32)
    out = A.decode(q, kp, vp, table, ctx, 0.3, "f32")
    for h in range(4):
        assert np.array_equal(out[0, h], v[0, h // 2].astype(np.float64))


def test_zero_query_gives_the_mean_of_v():
    rng = np.random.default_rng(2)
    k, v, kp, vp, table, ctx = tiny_pool(rng, 37)
    out = A.decode(np.zeros((1, 1, 32), np.float32), kp, vp, table, ctx, 0.5, "f32")
    np.testing.assert_allclose(out[0, 0], v[:, 0].astype(np.float64).mean(0), rtol=0, atol=1e-14)


@pytest.mark.parametrize("hot", [0, 15, 16, 36])
def test_dominant_key_selects_its_value(hot):
    rng = np.random.default_rng(4)
    k, v, kp, vp, table, ctx = tiny_pool(rng, 37)
    # rebuild with K = e_0 on the hot token and 0 elsewhere, then a huge q_0
    ks = [np.zeros((37, 1, 32), np.float32)]
    ks[0][hot, 0, 0] = 1.0
    kp, vp, table, ctx, _ = paged_from_logical(ks, [v], 5, "f32", rng.permutation(5), fill=np.nan)
    q = np.zeros((1, 1, 32), np.float32)
    q[0, 0, 0] = 1e4
    out = A.decode(q, kp, vp, table, ctx, 1.0, "f32")
    assert np.array_equal(out[0, 0], v[hot, 0].astype(np.float64))


def test_two_token_softmax_is_a_logistic_mix():
    rng = np.random.default_rng(6)
    k, v, kp, vp, table, ctx = tiny_pool(rng, 2)
    q = rng.standard_normal((1, 1, 32)).astype(np.float32)
    s = 0.7
    out = A.decode(q, kp, vp, table, ctx, s, "f32")
    z0 = s * float(np.dot(q[0, 0].astype(np.float64), k[0, 0].astype(np.float64)))
    z1 = s * float(np.dot(q[0, 0].astype(np.float64), k[1, 0].astype(np.float64)))
    w0 = 1 / (1 + math.exp(z1 - z0))
    want = w0 * v[0, 0].astype(np.float64) + (1 - w0) * v[1, 0].astype(np.float64)
    np.testing.assert_allclose(out[0, 0], want, rtol=0, atol=1e-14)


def test_query_heads_read_their_contiguous_kv_group():
    # Hq = 8, Hkv = 2: heads 0-3 read kv head 0, heads 4-7 read kv head 1
    n, D = 9, 32
    ks = [np.zeros((n, 2, D), np.float32)]
    vs = [np.zeros((n, 2, D), np.float32)]
    vs[0][:, 0, :] = 1.0
    vs[0][:, 1, :] = 2.0
    kp, vp, table, ctx, _ = paged_from_logical(ks, vs, 3, "f32", [2, 0, 1])
    q = np.random.default_rng(0).standard_normal((1, 8, D)).astype(np.float32)
    out = A.decode(q, kp, vp, table, ctx, 1.0, "f32")
    np.testing.assert_allclose(out[0, :4], 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(out[0, 4:], 2.0, rtol=0, atol=1e-14)


def test_scale_multiplies_the_scores():
    rng = np.random.default_rng(8)
    k, v, kp, vp, table, ctx = tiny_pool(rng, 30)
    q = rng.standard_normal((1, 1, 32)).astype(np.float32)
    a = A.decode(q * 2, kp, vp, table, ctx, 0.25, "f32")
    b = A.decode(q, kp, vp, table, ctx, 0.5, "f32")
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_zero_context_gives_zero_output():
    kp = np.full((2, 1, 16 * 32), np.nan, np.float32)
    out = A.decode(np.ones((1, 1, 32), np.float32), kp, kp, np.array([[0]]), np.array([0]), 1.0, "f32")
    assert np.array_equal(out, np.zeros((1, 1, 32)))


# ---------------------------------------------------------------- paging invariance

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_relabelling_physical_blocks_changes_nothing(dtype):
    w = make_workload("tiny_f32") if dtype == "f32" else make_workload("gqa8b_bf16", num_seqs=3, hi=100)
    bm = RefBlockManager(w.num_blocks, free_order=w.free_order)
    run_program(bm, w.program)
    table, ctx = bm.block_table(w.batch, w.max_blocks_per_seq(), pad=0)
    table, ctx = np.array(table), np.array(ctx)
    base = A.decode(w.decode_q, w.k_pool, w.v_pool, table, ctx, w.scale, w.dtype)
    perm = np.random.default_rng(9).permutation(w.num_blocks)
    kp = np.empty_like(w.k_pool)
    vp = np.empty_like(w.v_pool)
    kp[perm] = w.k_pool
    vp[perm] = w.v_pool
    moved = A.decode(w.decode_q, kp, vp, perm[table], ctx, w.scale, w.dtype)
    assert np.array_equal(base, moved)


def test_shared_prefix_equals_private_copies():
    w = make_workload("shared_prefix_bf16", num_users=6, num_prompts=2, user_tail=(16, 60))
    bm = RefBlockManager(w.num_blocks, free_order=w.free_order)
    run_program(bm, w.program)
    table, ctx = bm.block_table(w.batch, w.max_blocks_per_seq(), pad=0)
    table, ctx = np.array(table), np.array(ctx)
    base = A.decode(w.decode_q, w.k_pool, w.v_pool, table, ctx, w.scale, w.dtype)
    # give every sequence private copies of every block it uses
    used = sum(-(-int(c) // 16) for c in ctx)
    kp = np.concatenate([w.k_pool, np.zeros((used,) + w.k_pool.shape[1:], w.k_pool.dtype)])
    vp = np.concatenate([w.v_pool, np.zeros((used,) + w.v_pool.shape[1:], w.v_pool.dtype)])
    nxt = w.num_blocks
    private = table.copy()
    for s, c in enumerate(ctx):
        for j in range(-(-int(c) // 16)):
            kp[nxt] = w.k_pool[table[s, j]]
            vp[nxt] = w.v_pool[table[s, j]]
            private[s, j] = nxt
            nxt += 1
    assert len(set(table[:6, :4].ravel().tolist())) == 4  # the users really share 4 blocks
    assert np.array_equal(base, A.decode(w.decode_q, kp, vp, private, ctx, w.scale, w.dtype))


def test_unread_table_entries_and_tail_slots_do_not_matter():
    rng = np.random.default_rng(12)
    ks, vs = random_logical(rng, [21], 1, 32, "f32")
    kp, vp, table, ctx, _ = paged_from_logical(ks, vs, 4, "f32", [3, 1, 0, 2], fill=np.nan)
    padded = np.concatenate([table, np.array([[10 ** 9, -5]])], axis=1)
    q = rng.standard_normal((1, 1, 32)).astype(np.float32)
    out = A.decode(q, kp, vp, padded, ctx, 0.2, "f32")
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out[0, 0], brute_decode(q, ks, vs, 0.2, "f32")[0, 0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- chunk placement

def test_chunk_of_one_is_decode_and_rows_are_causal():
    rng = np.random.default_rng(13)
    lens, C = [50, 33], 6
    ks, vs = random_logical(rng, lens, 2, 32, "f16")
    kp, vp, table, ctx, _ = paged_from_logical(ks, vs, 12, "f16", rng.permutation(12), fill=np.nan)
    q = to_storage(rng.standard_normal((2, C, 4, 32), dtype=np.float32), "f16")
    pre = A.prefill_chunk(q, kp, vp, table, ctx, 0.3, "f16")
    # the last row is plain decode over the whole context
    np.testing.assert_array_equal(pre[:, -1], A.decode(q[:, -1], kp, vp, table, ctx, 0.3, "f16"))
    # row i equals decode over a context cut just after position ctx - C + i
    for i in range(C):
        cut = ctx - C + i + 1
        np.testing.assert_array_equal(pre[:, i], A.decode(q[:, i], kp, vp, table, cut, 0.3, "f16"))


# ---------------------------------------------------------------- tolerance feasibility

def test_tolerance_readings_hold_on_a_realistic_case():
    """bf16 output rounding alone exceeds a 1e-3 relative L2 budget, while the
    fp32 output of fp32 accumulation and a hi/lo split of p stays far below
    it; so the attention gate compares fp32 output, and p is never rounded to
    bf16 alone before the PV product."""
    w = make_workload("gqa8b_bf16", num_seqs=6, hi=1500)
    bm = RefBlockManager(w.num_blocks, free_order=w.free_order)
    run_program(bm, w.program)
    table, ctx = bm.block_table(w.batch, w.max_blocks_per_seq(), pad=0)
    ref = A.decode(w.decode_q, w.k_pool, w.v_pool, np.array(table), np.array(ctx), w.scale, "bf16")
    rel = lambda x: np.linalg.norm(x - ref) / np.linalg.norm(ref)  # noqa: E731
    assert rel(A.to_f64(A.round_f64_to(ref, "bf16"), "bf16")) > 1e-3
    assert rel(A.to_f64(A.round_f64_to(ref, "f16"), "f16")) < 1e-3
    assert rel(ref.astype(np.float32).astype(np.float64)) < 1e-6

    # p rounded once to bf16 before P.V, against the hi + lo split
    s = 0
    K, V = A.gather_kv(w.k_pool, w.v_pool, table[s], ctx[s], "bf16")
    qf = A.to_f64(w.decode_q[s, 0], "bf16")
    z = w.scale * (K[0] @ qf)
    p = np.exp(z - z.max())
    p = p / p.sum()
    exact = p @ V[0]
    bf = lambda x: A.to_f64(A.round_f64_to(x, "bf16"), "bf16")  # noqa: E731
    one = bf(p) @ V[0]
    hi = bf(p)
    two = hi @ V[0] + bf(p - hi) @ V[0]
    e1 = np.linalg.norm(one - exact) / np.linalg.norm(exact)
    e2 = np.linalg.norm(two - exact) / np.linalg.norm(exact)
    assert e1 > 1e-3 > 1e-5 > e2


# ------------------------------------------------- whole-block copies (CoW, swap)

def _labelled_pool(labels, codes, heads, run):
    """K and V pools whose block i holds label labels[i] (fixture rule)."""
    e = np.arange(run, dtype=np.float64)
    k = np.empty((len(labels), heads, run), dtype=np.float32)
    v = np.empty_like(k)
    for i, lab in enumerate(labels):
        for h in range(heads):
            k[i, h] = 1000 * (10 * codes[lab] + h) + e
            v[i, h] = 1000 * (10 * codes[lab] + h) + e + 500
    return k, v


def _assert_holds(k, v, labels, codes):
    want_k, want_v = _labelled_pool(labels, codes, k.shape[1], k.shape[2])
    assert np.array_equal(k, want_k)
    assert np.array_equal(v, want_v)


def test_copy_blocks_by_hand():
    g = load("block_copies_by_hand.txt")
    codes, H, run = g["label_codes"], g["num_kv_heads"], g["block_size"] * g["head_dim"]
    k, v = _labelled_pool(g["cow_pool"], codes, H, run)
    A.copy_blocks(k, v, np.array(g["cow_pairs"], dtype=np.int64))
    _assert_holds(k, v, g["cow_after"], codes)


def test_swap_blocks_by_hand():
    g = load("block_copies_by_hand.txt")
    codes, H, run = g["label_codes"], g["num_kv_heads"], g["block_size"] * g["head_dim"]
    dk, dv = _labelled_pool(g["swap_out_device"], codes, H, run)
    hk, hv = _labelled_pool(g["swap_out_host"], codes, H, run)
    A.swap_blocks(hk, hv, dk, dv, np.array(g["swap_out_pairs"], dtype=np.int64))
    _assert_holds(hk, hv, g["swap_out_host_after"], codes)
    _assert_holds(dk, dv, g["swap_out_device_after"], codes)
    A.swap_blocks(dk, dv, hk, hv, np.array(g["swap_in_pairs"], dtype=np.int64))
    _assert_holds(dk, dv, g["swap_in_device_after"], codes)
    _assert_holds(hk, hv, g["swap_in_host_after"], codes)
