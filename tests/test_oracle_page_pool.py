"""Pins the oracle allocator to hand-worked tables and to its invariants."""
import numpy as np
import pytest

from oracle.page_pool import OutOfPages, PagePool


def test_hand_worked_sequence_of_operations():
    pool = PagePool(8, [5, 2, 7, 0, 3, 6, 1, 4])
    assert pool.reserve(10, 20) == 2          # 20 tokens -> 2 blocks: pages 5, 2
    assert pool.reserve(11, 5) == 1           # page 7
    assert pool.reserve(10, 32) == 0          # still 2 blocks
    assert pool.reserve(10, 33) == 1          # third block: page 0
    assert pool.block_table([10, 11], 4).tolist() == [[5, 2, 0, -1], [7, -1, -1, -1]]
    pool.release(11)                          # page 7 goes to the back of the free list
    assert list(pool.free) == [3, 6, 1, 4, 7]
    assert pool.reserve(12, 48) == 3          # pages 3, 6, 1
    assert pool.block_table([12, 10], 3).tolist() == [[3, 6, 1], [5, 2, 0]]
    assert pool.num_free() == 2


def test_out_of_pages_changes_nothing():
    pool = PagePool(4, [3, 1, 0, 2])
    pool.reserve(1, 40)                       # 3 pages
    before = (list(pool.free), pool.blocks(1))
    with pytest.raises(OutOfPages):
        pool.reserve(1, 65)                   # needs 2 more, 1 free
    with pytest.raises(OutOfPages):
        pool.reserve(2, 17)
    assert (list(pool.free), pool.blocks(1)) == before and 2 not in pool.seqs


def test_tiny_workload_layout():
    # 32-page pool; sequence 0 holds 37 + 1 tokens (3 pages), sequence 1 holds 100 + 1 (7 pages).
    order = np.random.default_rng(0).permutation(32)
    pool = PagePool(32, order)
    pool.reserve(0, 38)
    pool.reserve(1, 101)
    bt = pool.block_table([0, 1], 7)
    assert bt[0, :3].tolist() == order[:3].tolist() and (bt[0, 3:] == -1).all()
    assert bt[1].tolist() == order[3:10].tolist()


def test_random_operations_keep_invariants():
    rng = np.random.default_rng(1)
    P = 64
    pool = PagePool(P, rng.permutation(P))
    lens = {}
    for _ in range(500):
        op = rng.integers(3)
        s = int(rng.integers(8))
        try:
            if op < 2:
                n = lens.get(s, 0) + int(rng.integers(0, 40))
                pool.reserve(s, n)
                lens[s] = n
            elif s in lens:
                pool.release(s)
                del lens[s]
        except OutOfPages:
            pass
        used = [p for pages in pool.seqs.values() for p in pages]
        assert len(used) == len(set(used))
        assert sorted(used + list(pool.free)) == list(range(P))
        for seq, n in lens.items():
            assert len(pool.blocks(seq)) == (n + 15) // 16


def test_fork_and_copy_on_write():
    pool = PagePool(6, [0, 1, 2, 3, 4, 5])
    pool.reserve(1, 20)                        # pages 0, 1 (block 1 holds tokens 16..19)
    pool.fork(1, 2)
    assert pool.blocks(2) == [0, 1] and pool.refs[0] == 2
    assert pool.reserve_for_write(2, 20) == (1, 2)   # shared last block -> fresh page 2
    assert pool.blocks(2) == [0, 2] and pool.blocks(1) == [0, 1]
    assert pool.reserve_for_write(2, 21) is None     # now private
    assert pool.reserve_for_write(1, 32) is None     # new block 2 for seq 1: page 3
    assert pool.blocks(1) == [0, 1, 3]
    pool.release(1)
    assert list(pool.free) == [4, 5, 1, 3] and pool.refs[0] == 1
    pool.release(2)
    assert sorted(pool.free) == list(range(6))
