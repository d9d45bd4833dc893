"""Pins for the allocator dict model (CPU only): the rules the pages state, worked by hand."""
import pytest

from oracle.allocator import OUT_OF_BLOCKS, AllocatorModel, AllocError


def _check(m):
    m.check_invariants()


def test_prefill_takes_ceil_blocks_and_slots_follow_the_table():
    m = AllocatorModel(10, 16)
    slots = m.seq_create(1, 40)
    blocks, n = m.seqs[1]
    assert n == 40 and len(blocks) == 3 and m.num_free == 7
    assert slots == [blocks[t // 16] * 16 + t % 16 for t in range(40)]
    _check(m)


def test_decode_append_fills_tail_then_takes_new_block():
    m = AllocatorModel(4, 16)
    m.seq_create(0, 15)
    s1, c1 = m.append([0])          # position 15 still in block 0
    assert c1 == [] and m.num_free == 3
    s2, c2 = m.append([0])          # position 16 needs a new block
    assert c2 == [] and m.num_free == 2
    b = m.seqs[0][0]
    assert s1 == [b[0] * 16 + 15] and s2 == [b[1] * 16]
    _check(m)


def test_fork_shares_blocks_and_counts_references():
    m = AllocatorModel(10, 16)
    m.seq_create(0, 40)
    m.fork(0, 1, 40)
    assert m.seqs[1][0] == m.seqs[0][0]
    assert all(m.ref[b] == 2 for b in m.seqs[0][0])
    assert m.num_free == 7
    _check(m)


def test_copy_on_write_of_shared_partial_tail():
    m = AllocatorModel(10, 16)
    m.seq_create(0, 40)              # tail block holds tokens 32..39
    m.fork(0, 1, 40)
    shared_tail = m.seqs[0][0][2]
    slots, cows = m.append([1])
    new_tail = m.seqs[1][0][2]
    assert cows == [(shared_tail, new_tail)] and new_tail != shared_tail
    assert slots == [new_tail * 16 + 8]
    assert m.seqs[0][0][2] == shared_tail          # the other sharer keeps the original
    assert m.ref[shared_tail] == 1 and m.ref[new_tail] == 1
    assert m.seqs[1][0][:2] == m.seqs[0][0][:2]   # full prefix blocks stay shared
    _check(m)
    # The last holder now owns it alone and writes in place.
    slots0, cows0 = m.append([0])
    assert cows0 == [] and slots0 == [shared_tail * 16 + 8]
    _check(m)


def test_all_sharers_appending_at_once_copy_all_but_the_last():
    m = AllocatorModel(20, 16)
    m.seq_create(0, 20)
    for c in (1, 2, 3):
        m.fork(0, c, 20)
    tail = m.seqs[0][0][1]
    assert m.ref[tail] == 4
    _, cows = m.append([0, 1, 2, 3])
    assert len(cows) == 3 and all(src == tail for src, _ in cows)
    assert m.ref[tail] == 1
    _check(m)


def test_full_shared_tail_needs_no_copy():
    m = AllocatorModel(10, 16)
    m.seq_create(0, 32)
    m.fork(0, 1, 32)
    _, cows = m.append([1])
    assert cows == []
    _check(m)


def test_exhaustion_fails_and_leaves_state_unchanged():
    m = AllocatorModel(3, 16)
    m.seq_create(0, 16)
    m.seq_create(1, 16)
    m.seq_create(2, 5)
    before = repr((m.free, m.ref, m.seqs))
    with pytest.raises(AllocError) as e:
        m.append([2, 0, 1])           # 2 fits in place, 0 and 1 each need a block
    assert e.value.status == OUT_OF_BLOCKS
    assert repr((m.free, m.ref, m.seqs)) == before
    with pytest.raises(AllocError):
        m.seq_create(9, 1)
    assert repr((m.free, m.ref, m.seqs)) == before


def test_free_returns_blocks_only_when_unreferenced():
    m = AllocatorModel(6, 16)
    m.seq_create(0, 48)
    m.fork(0, 1, 20)
    m.free_seq(0)
    assert m.num_free == 6 - 2       # the two blocks shared with 1 survive
    m.free_seq(1)
    assert m.num_free == 6
    _check(m)


def test_waste_stays_under_one_block():
    m = AllocatorModel(200, 16)
    for sid, L in enumerate([1, 15, 16, 17, 31, 32, 33, 100]):
        m.seq_create(sid, L)
        blocks, n = m.seqs[sid]
        assert 0 <= len(blocks) * 16 - n < 16
    _check(m)


def test_swap_out_and_back_keeps_length_and_unshares_blocks():
    dev, host = AllocatorModel(10, 4), AllocatorModel(6, 4)
    dev.seq_create(1, 10)          # blocks for tokens 0-3, 4-7, 8-9
    dev.fork(1, 2, 8)              # child shares the two full blocks
    free0 = len(dev.free)
    pairs = dev.swap_to(host, 1)
    assert len(pairs) == 3 and host.seqs[1][1] == 10
    assert [d for _, d in pairs] == host.seqs[1][0]
    assert all(host.ref[d] == 1 for _, d in pairs)
    # Only the block no one else holds returned to the device's free list.
    assert len(dev.free) == free0 + 1 and all(dev.ref[s] == 1 for s, _ in pairs[:2])
    back = host.swap_to(dev, 1)
    assert dev.seqs[1][1] == 10 and len(dev.seqs[1][0]) == 3
    # The swapped-in sequence owns fresh blocks; the child still holds the old shared ones.
    assert not set(dev.seqs[1][0]) & set(dev.seqs[2][0])
    assert [s for s, _ in back] == [d for _, d in pairs]     # read back from where it went
    _check(dev)
    _check(host)


def test_swap_exhaustion_fails_and_leaves_both_unchanged():
    dev, host = AllocatorModel(10, 4), AllocatorModel(2, 4)
    dev.seq_create(1, 9)
    snap = (list(dev.free), list(dev.ref), {k: (list(v[0]), v[1]) for k, v in dev.seqs.items()})
    with pytest.raises(AllocError) as e:
        dev.swap_to(host, 1)
    assert e.value.status == OUT_OF_BLOCKS
    assert (dev.free, dev.ref) == (snap[0], snap[1]) and dev.seqs[1] == [snap[2][1][0], 9]
    assert len(host.free) == 2 and not host.seqs


def test_stats_match_the_waste_closed_form():
    """Paged waste is sum over sequences of ceil(L/bs)*bs - L (each under one block); a
    fork adds logical blocks and tokens but no stored ones."""
    m = AllocatorModel(40, 16)
    lens = [1, 16, 17, 40]
    for i, L in enumerate(lens):
        m.seq_create(i, L)
    st = m.stats()
    assert st["used_blocks"] == 1 + 1 + 2 + 3 == st["logical_blocks"]
    assert st["tokens"] == st["stored_tokens"] == 74
    assert st["used_blocks"] * 16 - st["stored_tokens"] == 15 + 0 + 15 + 8
    m.fork(3, 9, 32)                       # shares the two full blocks of sequence 3
    st2 = m.stats()
    assert st2["used_blocks"] == 7 and st2["shared_blocks"] == 2 and st2["logical_blocks"] == 9
    assert st2["tokens"] == 74 + 32 and st2["stored_tokens"] == 74
    m.extend(9, 3)                         # the child writes past its shared prefix
    st3 = m.stats()
    assert st3["used_blocks"] == 8 and st3["stored_tokens"] == 77 and st3["free_blocks"] == 32
    _check(m)
