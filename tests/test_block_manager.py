"""Host block manager: pool, reference counts, sharing, copy-on-write decisions, slot placement.

Pinned against the pages' statements: waste at most BS - 1 slots per sequence, shared tables
point at one physical copy, a write into a shared still-filling block copies it first, freed
blocks return to the pool (and any free block fits any request).
"""
import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
import workloads
from workloads import BlockManager, PoolExhausted


def test_tiny_workload_waste_hits_both_extremes():
    case = workloads.tiny()
    bs = case.block_size
    waste = [(-(-int(L) // bs)) * bs - int(L) for L in case.context_lens]
    assert waste == [15, 1, 0, 15]
    assert waste == [oracle.paged_waste_slots(int(L), bs) for L in case.context_lens]


@settings(max_examples=60, deadline=None)
@given(lens=st.lists(st.integers(0, 700), min_size=1, max_size=12),
       bs=st.sampled_from([8, 16, 32, 64]))
def test_waste_at_most_block_size_minus_one(lens, bs):
    need = sum(-(-L // bs) for L in lens)
    bm = BlockManager(need + 3, bs, free_order=np.random.default_rng(0).permutation(need + 3))
    for L in lens:
        bm.new_sequence(L)
    for s, L in enumerate(lens):
        assert 0 <= bm.waste_slots(s) <= bs - 1
        assert bm.waste_slots(s) == oracle.paged_waste_slots(L, bs)
    assert bm.num_free == 3


@settings(max_examples=40, deadline=None)
@given(lens=st.lists(st.integers(1, 200), min_size=1, max_size=8), steps=st.integers(1, 40),
       bs=st.sampled_from([8, 16]))
def test_appends_place_tokens_in_unique_slots_consistent_with_tables(lens, steps, bs):
    nb = sum(-(-(L + steps) // bs) for L in lens) + 2
    bm = BlockManager(nb, bs, free_order=np.random.default_rng(1).permutation(nb))
    for L in lens:
        bm.new_sequence(L)
    seen = set()
    for _ in range(steps):
        before = list(bm.lens)
        plan = bm.append_tokens(range(len(lens)))
        assert plan.block_mapping.shape == (0, 2)  # nothing shared, nothing copied
        for s, slot in zip(plan.seq_ids, plan.slot_mapping):
            pos = before[s]
            assert slot == bm.tables[s][pos // bs] * bs + pos % bs
            assert slot not in seen
            seen.add(int(slot))
    for s, L in enumerate(lens):
        assert bm.lens[s] == L + steps
        assert len(bm.tables[s]) == -(-(L + steps) // bs)


def test_fork_then_append_copies_once_and_repoints():
    bm = BlockManager(10, 4, free_order=list(range(10)))
    a = bm.new_sequence(6)  # blocks 0, 1 (block 1 holds 2 of 4 slots)
    b = bm.fork(a)
    assert bm.tables[a] == bm.tables[b] == [0, 1]
    assert list(bm.refcount[:2]) == [2, 2]
    plan = bm.append_tokens([a, b])
    # a writes into shared, still-filling block 1 -> copy 1 -> 2, re-point a; b writes in place
    assert plan.block_mapping.tolist() == [[1, 2]]
    assert bm.tables[a] == [0, 2] and bm.tables[b] == [0, 1]
    assert plan.slot_mapping.tolist() == [2 * 4 + 2, 1 * 4 + 2]
    assert list(bm.refcount[:3]) == [2, 1, 1]


def test_full_last_block_allocates_instead_of_copying():
    bm = BlockManager(10, 4, free_order=list(range(10)))
    a = bm.new_sequence(8)
    bm.fork(a)
    plan = bm.append_tokens([0, 1])
    assert plan.block_mapping.shape == (0, 2)
    assert bm.tables[0] == [0, 1, 2] and bm.tables[1] == [0, 1, 3]


def test_prefix_sharing_counts_and_free_returns_blocks():
    bm = BlockManager(40, 16, free_order=list(range(40)))
    prefix = bm.reserve(2)
    seqs = [bm.new_sequence(32 + 5 * i + 1, prefix=prefix) for i in range(5)]
    assert all(bm.tables[s][:2] == prefix for s in seqs)
    assert bm.refcount[prefix[0]] == 6
    free_before = bm.num_free
    bm.free_sequence(seqs[0])
    assert bm.num_free == free_before + 1  # only its private block comes back
    assert bm.refcount[prefix[0]] == 5


def test_pool_exhaustion_raises():
    bm = BlockManager(3, 16)
    bm.new_sequence(48)
    with pytest.raises(PoolExhausted):
        bm.new_sequence(1)


def test_shared_prefix_fork_workload_plan():
    case = workloads.shared_prefix(True)
    st_ = case.step
    lens = st_.pre_context_lens
    # every sibling pair whose last block is partially filled issues exactly one copy
    expect = sum(1 for L in lens[::2] if L % 16)
    assert len(st_.block_mapping) == expect
    workloads.check_plan(workloads.AppendPlan(st_.block_mapping, st_.slot_mapping, []), 16)
