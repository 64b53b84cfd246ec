"""The host block manager (include/paged_block_manager.h): the operations of
page "paged-attention-runtime" (BlockManager: free list, reference counts,
allocate_blocks, free_sequence, share_prefix, cow_block), checked by their
stated effects and by invariants of the manager's own reported state under
random operation sequences. CPU only."""
import numpy as np
import pytest

import paged_gqa_decode_block_amd as pa
from paged_gqa_decode_block_amd import workload as W


def state(bm, seqs):
    """(free count, ref counts, block lists) as the manager reports them."""
    return (bm.num_free, [bm.ref_count(b) for b in range(bm.num_blocks)],
            {s: bm.sequence_blocks(s) for s in seqs})


def check_invariants(bm, seqs):
    free, refs, lists = state(bm, seqs)
    uses = np.zeros(bm.num_blocks, dtype=np.int64)
    for s, blocks in lists.items():
        assert len(set(blocks)) == len(blocks), f"sequence {s} lists a block twice"
        for b in blocks:
            uses[b] += 1
    assert list(uses) == refs, "a reference count differs from the number of lists holding the block"
    assert free + int((uses > 0).sum()) == bm.num_blocks, "free + used != pool"


def test_operations_as_the_page_states():
    bm = pa.BlockManager(12, 16)
    assert bm.num_free == 12
    bm.allocate_blocks(7, 3)
    assert bm.sequence_blocks(7) == [0, 1, 2] and bm.num_free == 9
    assert all(bm.ref_count(b) == 1 for b in (0, 1, 2))
    bm.share_prefix(7, 8, 2)                       # prefix sharing raises ref counts
    assert bm.sequence_blocks(8) == [0, 1]
    assert (bm.ref_count(0), bm.ref_count(1), bm.ref_count(2)) == (2, 2, 1)
    assert bm.num_free == 9                        # nothing allocated by sharing
    assert bm.cow_block(7, 2) is None              # exclusive: nothing to copy
    src, dst = bm.cow_block(8, 1)                  # shared: a fresh block replaces it
    assert src == 1 and dst not in (0, 1, 2)
    assert bm.sequence_blocks(8) == [0, dst] and bm.ref_count(1) == 1 and bm.ref_count(dst) == 1
    bm.free_sequence(7)                            # blocks return at zero references
    assert bm.ref_count(0) == 1 and bm.ref_count(1) == 0 and bm.ref_count(2) == 0
    assert bm.num_free == 12 - 2
    bm.free_sequence(8)
    assert bm.num_free == 12 and all(bm.ref_count(b) == 0 for b in range(12))


def test_append_slot_allocates_and_copies_on_write():
    bm = pa.BlockManager(8, 4)
    assert bm.append_slot(1, 0) is None and bm.sequence_blocks(1) == [0]
    for t in (1, 2, 3):
        assert bm.append_slot(1, t) is None and bm.sequence_blocks(1) == [0]
    assert bm.append_slot(1, 4) is None and bm.sequence_blocks(1) == [0, 1]
    bm.share_prefix(1, 2, 2)                      # 2 shares both blocks (token 5 is next)
    src, dst = bm.append_slot(2, 5)               # writing into the shared last block
    assert src == 1 and bm.sequence_blocks(2) == [0, dst]
    assert bm.append_slot(1, 5) is None           # block 1 is 1's alone now
    with pytest.raises(pa.PagedAttnError):
        bm.append_slot(1, 12)                     # a gap: blocks for tokens 8..11 missing
    check_invariants(bm, [1, 2])


def test_block_table_layout():
    bm = pa.BlockManager(6, 16)
    bm.allocate_blocks(10, 2)
    bm.allocate_blocks(11, 1)
    bm.share_prefix(10, 12, 1)
    t = bm.block_table([11, 10, 12], 3)
    assert t.dtype == np.int32 and t.tolist() == [[2, -1, -1], [0, 1, -1], [0, -1, -1]]
    with pytest.raises(pa.PagedAttnError):
        bm.block_table([10], 1)                   # more blocks than max_blocks_per_seq
    with pytest.raises(pa.PagedAttnError):
        bm.block_table([99], 4)                   # unknown sequence


def test_failed_operations_change_nothing():
    bm = pa.BlockManager(5, 16)
    bm.allocate_blocks(1, 3)
    bm.share_prefix(1, 2, 3)
    before = state(bm, [1, 2])
    for op in (lambda: bm.allocate_blocks(3, 3),      # only 2 free
               lambda: bm.free_sequence(9),
               lambda: bm.share_prefix(1, 2, 1),       # target exists
               lambda: bm.share_prefix(1, 4, 4),       # source too short
               lambda: bm.cow_block(1, 3),             # index out of range
               lambda: bm.allocate_blocks(1, -1)):
        with pytest.raises(pa.PagedAttnError):
            op()
        assert state(bm, [1, 2]) == before
    bm.allocate_blocks(3, 2)                           # the pool is now full
    before = state(bm, [1, 2, 3])
    with pytest.raises(pa.PagedAttnError):
        bm.cow_block(2, 0)                             # shared, but no free block
    assert state(bm, [1, 2, 3]) == before
    assert pa.strerror(-14) and pa.strerror(-15)


def test_random_operation_sequences_keep_invariants():
    rng = np.random.default_rng(17)
    bm = pa.BlockManager(64, 8)
    live, next_id = [], 0
    for _ in range(3000):
        op = rng.integers(0, 6)
        before = state(bm, live)
        try:
            if op == 0 or not live:
                n = int(rng.integers(0, 6))
                free = bm.num_free
                bm.allocate_blocks(next_id, n)
                assert bm.num_free == free - n and len(bm.sequence_blocks(next_id)) == n
                live.append(next_id)
                next_id += 1
            elif op == 1:
                s = live.pop(int(rng.integers(0, len(live))))
                bm.free_sequence(s)
            elif op == 2:
                s = live[int(rng.integers(0, len(live)))]
                blocks = bm.sequence_blocks(s)
                n = int(rng.integers(0, len(blocks) + 1))
                bm.share_prefix(s, next_id, n)
                assert bm.sequence_blocks(next_id) == blocks[:n]
                live.append(next_id)
                next_id += 1
            elif op == 3:
                s = live[int(rng.integers(0, len(live)))]
                blocks = bm.sequence_blocks(s)
                if blocks:
                    i = int(rng.integers(0, len(blocks)))
                    shared = bm.ref_count(blocks[i]) > 1
                    r = bm.cow_block(s, i)
                    assert (r is not None) == shared
                    if r:
                        assert r[0] == blocks[i] and before[1][r[1]] == 0
                        assert bm.ref_count(r[0]) == before[1][r[0]] - 1
                        assert bm.sequence_blocks(s) == blocks[:i] + [r[1]] + blocks[i + 1:]
            elif op == 4:
                s = live[int(rng.integers(0, len(live)))]
                blocks = bm.sequence_blocks(s)
                t = len(blocks) * bm.block_size - int(rng.integers(0, bm.block_size + 1))
                bm.append_slot(s, max(t, 0))
            else:
                s = live[int(rng.integers(0, len(live)))]
                bm.allocate_blocks(s, int(rng.integers(1, 3)))
        except pa.PagedAttnError:
            assert state(bm, live) == before
        check_invariants(bm, live)


def test_prefix_shared_workload_structure():
    """The prefix-shared decode workload built with the manager: 16 families of
    16 sequences whose first 64 blocks are shared (the last sequence of the last
    family holds only the first prefix block). Reference counts match the
    workload generator's."""
    case = W.make_config(5, tables_only=True)
    bs = case.bs
    bm = pa.BlockManager(case.NB, bs)
    seqs = []
    fam = 16
    for f in range(16):
        head = f * fam
        for i in range(fam):
            s = head + i
            L = int(case.seqlens[s])
            if i == 0:
                bm.allocate_blocks(s, -(-L // bs))
            else:
                shared = min(64, -(-L // bs))
                bm.share_prefix(head, s, shared)
                bm.allocate_blocks(s, -(-L // bs) - shared)
            seqs.append(s)
    table = bm.block_table(seqs, case.MBS)
    refs = np.array([bm.ref_count(b) for b in range(case.NB)])
    got = np.bincount(refs, minlength=17)
    want = np.bincount(case.ref_count, minlength=17)
    assert list(got) == list(want)
    # every sequence's row lists ceil(L / bs) blocks, -1 after
    for s in seqs:
        n = -(-int(case.seqlens[s]) // bs)
        assert (table[s, :n] >= 0).all() and (table[s, n:] == -1).all()
    check_invariants(bm, seqs)
