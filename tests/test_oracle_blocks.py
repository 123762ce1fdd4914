"""The block bookkeeping model pinned to what the pages state about the
allocator, the per-block counts and rollback, and to invariants that any
correct bookkeeping keeps."""
import random

import pytest

from oracle.blocks import Blocks, Exhausted


def check_invariants(m: Blocks):
    refs = [0] * m.num_blocks
    for length, table in m.seqs.values():
        assert len(table) == -(-length // m.block_size)     # the table covers exactly the length
        for b in table:
            refs[b] += 1
    assert refs == m.count                                  # a count is the number of owners
    assert sorted(m.free) == [b for b in range(m.num_blocks) if m.count[b] == 0]
    assert len(set(m.free)) == len(m.free)


def test_page_zero_first_and_slots():
    m = Blocks(8, 4)
    s = m.seq_new()
    slots, cow = m.append(s, 10)
    assert cow == (-1, -1)
    assert m.seqs[s][1] == [0, 1, 2]                        # the reversed stack hands out 0, 1, 2
    assert slots == list(range(10))                         # block * 4 + offset
    t = m.seq_new()
    slots, _ = m.append(t, 1)
    assert slots == [12] and len(m.free) == 4


def test_popn_frees_trailing_pages_only():
    m = Blocks(8, 4)
    s = m.seq_new()
    m.append(s, 10)                                         # pages 0, 1, 2 (2 half full)
    assert m.popn(s, 1) == 1 and m.seqs[s][1] == [0, 1, 2]  # 9 positions still need 3 pages
    assert m.popn(s, 1) == 1 and m.seqs[s][1] == [0, 1]     # 8 positions: page 2 freed
    assert m.free[-1] == 2                                  # and handed out next
    assert m.popn(s, 100) == 8 and m.seqs[s] == [0, []]     # at most the length
    check_invariants(m)


def test_exhaustion_changes_nothing():
    m = Blocks(3, 4)
    s = m.seq_new()
    m.append(s, 5)
    before = (list(m.free), list(m.count), {k: [v[0], list(v[1])] for k, v in m.seqs.items()})
    with pytest.raises(Exhausted):
        m.append(s, 8)                                      # needs 2 more pages, 1 left
    assert (m.free, m.count, m.seqs) == before
    m.append(s, 7)                                          # exactly fits
    assert m.free == []


def test_fork_shares_and_copies_on_write():
    m = Blocks(8, 4)
    p = m.seq_new()
    m.append(p, 6)                                          # pages 0, 1 (1 half full)
    c = m.seq_fork(p)
    assert m.count[0] == m.count[1] == 2 and m.seqs[c] == [6, [0, 1]]
    slots, cow = m.append(c, 1)                             # writes into shared page 1
    assert cow == (1, 2) and m.seqs[c][1] == [0, 2] and slots == [2 * 4 + 2]
    assert m.count[1] == 1 and m.seqs[p][1] == [0, 1]       # the parent keeps page 1
    slots, cow = m.append(p, 2)                             # page 1 is the parent's alone now
    assert cow == (-1, -1) and slots == [6, 7]
    check_invariants(m)


def test_fork_at_a_page_boundary_needs_no_copy():
    m = Blocks(8, 4)
    p = m.seq_new()
    m.append(p, 8)
    c = m.seq_fork(p)
    slots, cow = m.append(c, 3)
    assert cow == (-1, -1) and m.seqs[c][1] == [0, 1, 2] and slots == [8, 9, 10]
    m.seq_free(p)
    assert m.count[0] == m.count[1] == 1 and sorted(m.free) == [3, 4, 5, 6, 7]
    check_invariants(m)


def test_free_reuses_lowest_id_and_returns_last_block_first():
    m = Blocks(8, 2)
    a, b = m.seq_new(), m.seq_new()
    m.append(a, 5)                                          # pages 0, 1, 2
    m.seq_free(a)
    assert m.free[-3:] == [2, 1, 0] and m.seq_new() == a    # page 0 comes out first again
    assert b == 1


def test_random_operations_keep_the_invariants():
    rng = random.Random(7)
    m = Blocks(40, 4)
    for _ in range(3000):
        op = rng.random()
        live = sorted(m.seqs)
        try:
            if op < 0.15 or not live:
                m.seq_new()
            elif op < 0.25:
                m.seq_fork(rng.choice(live))
            elif op < 0.35:
                m.seq_free(rng.choice(live))
            elif op < 0.75:
                s = rng.choice(live)
                slots, cow = m.append(s, rng.randint(0, 9))
                # a write never lands in a block another sequence still holds
                assert all(m.count[x // 4] == 1 for x in slots)
            else:
                m.popn(rng.choice(live), rng.randint(0, 9))
        except Exhausted:
            pass
        check_invariants(m)
