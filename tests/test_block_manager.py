"""The host block manager: pins of the oracle (oracle/block_manager.py)
against the pages, planted mistakes that the pins catch, the same pins on
the native manager, and bit-exact parity of the native manager
(libpagedkv.so, C ABI) with the oracle over random operation sequences.
CPU only: the manager is host code."""
import random

import numpy as np
import pytest

import oracle as O
from oracle.block_manager import BlockManagerOracle
from paged_attention_decode_scatter_amd import native as N
from tests.conftest import golden


# ---------------------------------------------------------------------------
# pins of the oracle
# ---------------------------------------------------------------------------
def pin_thirty_tokens(cls):
    """mini-runtime ch. 12, 7 (exercise): 30 tokens at block size 16 take 2
    blocks with the last 14/16 full; at block size 4, 8 blocks, last 2/4."""
    g = golden("p3_think_30_tokens.json")
    for case in g["cases"]:
        bs = case["block_size"]
        m = cls(64, bs)
        assert m.allocate(0, 30)
        assert len(m.table(0)) == case["blocks"]
        st = m.stats()
        assert st["used"] == case["blocks"]
        last_fill = 30 - (case["blocks"] - 1) * bs
        assert last_fill == case["last_block_tokens"]
        assert st["utilization"] == pytest.approx(30 / (case["blocks"] * bs))


def pin_short_queue_takes_nothing(cls):
    """ch. 12, 2.3: allocate answers False when the free queue cannot cover
    ceil(num_tokens / bs) blocks, and takes nothing."""
    m = cls(4, 16)
    assert m.allocate(1, 40)              # 3 blocks
    before = list(m.free_ids)
    assert not m.can_allocate(17)           # needs 2, 1 free
    assert m.allocate(2, 17) is False
    assert list(m.free_ids) == before and 2 not in m.seqs
    assert m.allocate(3, 16)              # exactly 1 block fits


def pin_fifo_order(cls):
    """ch. 12, 2.3 and 4.2: blocks come from the left of a FIFO queue in
    order; freed blocks join it at the right."""
    m = cls(8, 16)
    assert m.allocate(1, 40)
    assert m.table(1) == [0, 1, 2]
    assert m.allocate(2, 20)
    assert m.table(2) == [3, 4]
    m.free(1)
    assert list(m.free_ids) == [5, 6, 7, 0, 1, 2]
    assert m.allocate(3, 64)
    assert m.table(3) == [5, 6, 7, 0]


def pin_ref_count_release(cls):
    """ch. 12, 2.4: a block shared by two holders goes back to the free
    queue only when the last holder leaves."""
    m = cls(8, 16)
    assert m.allocate(1, 48)
    m.share(1, 2, 2)
    assert m.ref_count[:3] == [2, 2, 1]
    m.free(1)
    assert 0 not in m.free_ids and 1 not in m.free_ids and 2 in m.free_ids
    m.free(2)
    assert 0 in m.free_ids and 1 in m.free_ids
    assert all(r == 0 for r in m.ref_count)


def pin_release_order(cls):
    """ch. 12, 7 (exercise): two requests holding a ref_count-2 block finish
    in either order -- the final state (free set, reference counts) is the
    same; only the queue order of the freed blocks differs."""
    def run(order):
        m = cls(8, 16)
        assert m.allocate(1, 48)
        m.share(1, 2, 2)
        assert m.append_slot(2) is not None    # b's own block
        for q in order:
            m.free(q)
        return m

    x, y = run([1, 2]), run([2, 1])
    assert sorted(x.free_ids) == sorted(y.free_ids) == list(range(8))
    assert x.ref_count == y.ref_count
    assert x.used() == y.used() == 0


def pin_append_slot(cls):
    """vLLM source notes 2.1: the decode append takes the next slot of the
    last block when it has room, a new block when it is full; the slot is
    the one of the slot formula (pinned separately) at the new position."""
    m = cls(16, 16)
    assert m.allocate(1, 14, offset=1)          # flat positions 1..14
    s = m.append_slot(1)                        # position 15: same block
    assert s == m.table(1)[0] * 16 + 15 and len(m.table(1)) == 1
    s = m.append_slot(1)                        # position 16: new block
    assert len(m.table(1)) == 2 and s == m.table(1)[1] * 16
    # against the slot formula of the C oracle
    bt = np.array([m.table(1) + [-1] * 4], dtype=np.int32)
    ref = O.slot_mapping(bt, np.array([1], np.int32), np.array([0], np.int32),
                         np.array([15], np.int32), 16)
    assert int(ref[0]) == s


def pin_capacity(cls):
    """ch. 12, 2.2: capacity = blocks * block_size - offset, and allocate
    takes just enough blocks for the tokens from the offset on."""
    for bs in (4, 16):
        for off in (0, 1, bs - 1):
            for n in (1, bs - off, bs - off + 1, 3 * bs):
                m = cls(64, bs)
                assert m.allocate(1, n, offset=off)
                cap = m.capacity(1)
                assert cap == len(m.table(1)) * bs - off
                assert n <= cap < n + bs


def pin_fragmentation(cls):
    """vLLM source notes, 3: only each sequence's last block is partly
    empty, so waste stays under 4 % for decode-length sequences."""
    rng = random.Random(3)
    m = cls(16384, 16)
    for i in range(32):
        assert m.allocate(i, rng.randint(128, 2048))
    assert 1 - m.stats()["utilization"] < 0.04


PINS = [pin_thirty_tokens, pin_short_queue_takes_nothing, pin_fifo_order, pin_ref_count_release,
        pin_release_order, pin_append_slot, pin_capacity, pin_fragmentation]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pins(pin):
    pin(BlockManagerOracle)


# ---------------------------------------------------------------------------
# copy-on-write (ch. 12, 3.1: sharing by copy-on-write + ref_count; 2.3 the
# FIFO take and its False; 2.4 reference counts)
# ---------------------------------------------------------------------------
def cow_state(m, seqs):
    return (list(m.free_ids), list(m.ref_count), {q: m.table(q) for q in seqs})


def pin_cow_unshared_is_noop(cls):
    """A block held by one table needs no copy: (b, b), nothing changes."""
    m = cls(6, 4)
    assert m.allocate(1, 10)
    before = cow_state(m, [1])
    b = m.table(1)[2]
    assert m.cow(1, 2) == (b, b)
    assert cow_state(m, [1]) == before


def pin_cow_moves_one_reference_to_the_fifo_front(cls):
    """The writer of a shared block takes the free queue's front block in
    its table, the old block keeps its other holder, counts 1 and 1."""
    m = cls(8, 4)
    assert m.allocate(1, 12)          # blocks 0, 1, 2
    m.share(1, 2, 2)                  # 2 holds 0, 1 (counts 2, 2, 1)
    front = m.free_ids[0]
    t1 = m.table(1)
    assert m.cow(2, 1) == (t1[1], front)
    assert m.table(2) == [t1[0], front] and m.table(1) == t1
    assert m.ref_count[t1[1]] == 1 and m.ref_count[front] == 1 and m.ref_count[t1[0]] == 2
    assert front not in m.free_ids


def pin_cow_short_queue_changes_nothing(cls):
    """Shared block, empty free queue: False, nothing taken or moved."""
    m = cls(3, 4)
    assert m.allocate(1, 12)          # all three blocks
    m.share(1, 2, 3)
    before = cow_state(m, [1, 2])
    assert m.cow(2, 0) is False
    assert cow_state(m, [1, 2]) == before


def pin_cow_then_free_returns_every_block(cls):
    """After copies, freeing every holder frees every block."""
    m = cls(10, 4)
    assert m.allocate(1, 16)
    m.share(1, 2, 4)
    m.share(1, 3, 2)
    for q, j in [(2, 3), (3, 0), (3, 1), (2, 0)]:
        assert m.cow(q, j)
    for q in (1, 2, 3):
        m.free(q)
    assert all(r == 0 for r in m.ref_count) and sorted(m.free_ids) == list(range(10))


def pin_cow_then_append_writes_the_private_block(cls):
    """A sequence sharing a partly filled last block copies it and then
    appends into its own copy, not into the shared one."""
    m = cls(8, 4)
    assert m.allocate(1, 6)           # blocks 0, 1; block 1 holds 2 tokens
    m.share(1, 2, 2)                  # 2 holds the same 8 slots; len 8
    m2_last = m.table(2)[1]
    old, new = m.cow(1, 1)
    assert old == m2_last and new != old
    slot = m.append_slot(1)           # token 6 of sequence 1
    assert slot // 4 == new and slot % 4 == 2


COW_PINS = [pin_cow_unshared_is_noop, pin_cow_moves_one_reference_to_the_fifo_front,
            pin_cow_short_queue_changes_nothing, pin_cow_then_free_returns_every_block,
            pin_cow_then_append_writes_the_private_block]


@pytest.mark.parametrize("pin", COW_PINS, ids=lambda f: f.__name__)
def test_oracle_cow_pins(pin):
    pin(BlockManagerOracle)


class _CowKeepsOldReference(BlockManagerOracle):
    def cow(self, seq, index):
        st = self.seqs[seq]
        b = st["blocks"][index]
        if self.ref_count[b] <= 1:
            return (b, b)
        if not self.free_ids:
            return False
        nb = self.free_ids.popleft()
        self.ref_count[nb] = 1
        st["blocks"][index] = nb
        return (b, nb)


class _CowFromTheBack(BlockManagerOracle):
    def cow(self, seq, index):
        if self.free_ids:
            self.free_ids.rotate(-1)  # the back id comes to the front
        return super().cow(seq, index)


class _CowAlwaysCopies(BlockManagerOracle):
    def cow(self, seq, index):
        st = self.seqs[seq]
        b = st["blocks"][index]
        if not self.free_ids:
            return False
        self.ref_count[b] += 1
        return super().cow(seq, index)


@pytest.mark.parametrize("mutant", [_CowKeepsOldReference, _CowFromTheBack, _CowAlwaysCopies],
                         ids=lambda c: c.__name__)
def test_planted_cow_mistake_fails_a_pin(mutant):
    failed = 0
    for pin in COW_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError, IndexError, KeyError, TypeError):
            failed += 1
    assert failed > 0


# Plausible mistakes planted in copies of the oracle: each must fail a pin.
class _Lifo(BlockManagerOracle):
    def dec_ref(self, block):
        self.ref_count[block] -= 1
        if self.ref_count[block] == 0:
            self.free_ids.appendleft(block)


class _FreeOnFirstRelease(BlockManagerOracle):
    def dec_ref(self, block):
        self.ref_count[block] = 0
        if block not in self.free_ids:
            self.free_ids.append(block)


class _FloorBlocks(BlockManagerOracle):
    def blocks_for(self, num_tokens, offset=0):
        return (offset + num_tokens) // self.block_size


class _AppendIgnoresOffset(BlockManagerOracle):
    def append_slot(self, seq):
        st = self.seqs[seq]
        off = st["offset"]
        st["offset"] = 0
        try:
            return super().append_slot(seq)
        finally:
            st["offset"] = off


class _PartialTake(BlockManagerOracle):
    def allocate(self, seq, num_tokens, offset=0):
        need = self.blocks_for(num_tokens, offset)
        blocks = []
        while self.free_ids and len(blocks) < need:
            b = self.free_ids.popleft()
            self.ref_count[b] = 1
            blocks.append(b)
        self.seqs[seq] = {"blocks": blocks, "offset": offset, "len": num_tokens}
        self._note_peak()
        return len(blocks) == need


@pytest.mark.parametrize("mutant", [_Lifo, _FreeOnFirstRelease, _FloorBlocks,
                                    _AppendIgnoresOffset, _PartialTake],
                         ids=lambda c: c.__name__)
def test_planted_mistake_fails_a_pin(mutant):
    failed = 0
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError, IndexError, KeyError, TypeError):
            failed += 1
    assert failed > 0


# ---------------------------------------------------------------------------
# the native manager
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_native_meets_the_pins(pin):
    pin(N.BlockManager)


@pytest.mark.parametrize("pin", COW_PINS, ids=lambda f: f.__name__)
def test_native_meets_the_cow_pins(pin):
    pin(N.BlockManager)


def state(m, seqs):
    tabs = {q: m.table(q) for q in sorted(seqs)}
    st = m.stats()
    return (list(m.free_ids), list(m.ref_count), tabs,
            {q: (m.seqs[q]["len"] if isinstance(m, BlockManagerOracle) else m.seq_len(q))
             for q in sorted(seqs)},
            (st["free"], st["used"], st["peak_used"], st["live_tokens"]))


@pytest.mark.parametrize("seed", range(12))
def test_native_matches_oracle_on_random_operations(seed):
    """allocate (with offsets), share, append_slot, copy-on-write, free,
    inc_ref / dec_ref in random order, driven to shortage; after every operation the free
    queue, the reference counts, every table and length, and the statistics
    are identical, and so are the answers (success, slots)."""
    rng = random.Random(seed)
    bs = rng.choice([1, 4, 16])
    nb = rng.choice([6, 24, 96])
    o, n = BlockManagerOracle(nb, bs), N.BlockManager(nb, bs)
    live, extra, next_id = set(), [], 0
    for _ in range(400):
        op = rng.random()
        if op < 0.25 or not live:
            ln = rng.randint(0, 5 * bs)
            off = rng.randrange(bs)
            assert o.can_allocate(ln, off) == n.can_allocate(ln, off)
            r = o.allocate(next_id, ln, off)
            assert n.allocate(next_id, ln, off) == r
            if r:
                live.add(next_id)
            next_id += 1
        elif op < 0.35:
            src = rng.choice(sorted(live))
            k = len(o.table(src))
            if k:
                j = rng.randint(1, k)
                o.share(src, next_id, j)
                n.share(src, next_id, j)
                live.add(next_id)
                next_id += 1
        elif op < 0.65:
            q = rng.choice(sorted(live))
            assert o.append_slot(q) == n.append_slot(q)
        elif op < 0.75:
            q = rng.choice(sorted(live))
            k = len(o.table(q))
            if k:
                j = rng.randrange(k)
                assert o.cow(q, j) == n.cow(q, j)
        elif op < 0.9:
            q = rng.choice(sorted(live))
            o.free(q)
            n.free(q)
            live.discard(q)
        elif op < 0.95:
            used = [b for b in range(nb) if o.ref_count[b] > 0]
            if used:
                b = rng.choice(used)
                o.inc_ref(b)
                n.inc_ref(b)
                extra.append(b)
        elif extra:
            b = extra.pop(rng.randrange(len(extra)))
            o.dec_ref(b)
            n.dec_ref(b)
        assert state(o, live) == state(n, live)


def test_native_batch_append_and_tables():
    m, o = N.BlockManager(10, 4), BlockManagerOracle(10, 4)
    for q, (ln, off) in enumerate([(3, 1), (4, 0), (9, 2)]):
        assert m.allocate(q, ln, off) and o.allocate(q, ln, off)
    k, slots = m.append_slots([0, 1, 2, 0])
    assert k == 4
    assert list(slots) == [o.append_slot(q) for q in [0, 1, 2, 0]]
    tab, lens, offs = m.tables([2, 0])
    assert list(lens) == [10, 5] and list(offs) == [2, 1]
    assert [b for b in tab[0] if b >= 0] == o.table(2) and tab.shape[1] == 3
    # shortage part-way: the appended prefix is reported, the rest untouched
    free = len(m.free_ids)
    big = list(range(3)) * 8
    k, slots = m.append_slots(big)
    assert k < len(big) and len(m.free_ids) == 0 and free > 0
    assert all(s >= 0 for s in slots[:k]) and all(s == -1 for s in slots[k:])


def test_native_argument_errors():
    m = N.BlockManager(4, 16)
    with pytest.raises(N.PagedKVError):
        m.allocate(0, 10, offset=16)
    assert m.allocate(0, 10)
    with pytest.raises(N.PagedKVError):
        m.allocate(0, 10)                 # exists
    with pytest.raises(N.PagedKVError):
        m.free(7)                         # unknown
    with pytest.raises(N.PagedKVError):
        m.dec_ref(3)                      # free block
    with pytest.raises(N.PagedKVError):
        m.share(0, 1, 2)                  # more blocks than src holds
    assert m.allocate(1, 100) is False    # short: not an error
    with pytest.raises(N.PagedKVError):
        m.cow(5, 0)                       # unknown sequence
    with pytest.raises(N.PagedKVError):
        m.cow(0, 1)                       # past the table
    with pytest.raises(N.PagedKVError):
        m.cow(0, -1)
    assert m.cow(0, 0) == (m.table(0)[0],) * 2
    lib = N.load_library()
    assert lib.pkv_bm_create(0, 16) is None
    assert N.status_string(N.NO_SPACE) == "too few free blocks (nothing changed)"
