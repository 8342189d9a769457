"""The host block manager: pins of the oracle (oracle/block_manager.py)
against the pages, and planted mistakes that the pins catch."""
import random

import numpy as np
import pytest

import oracle as O
from oracle.block_manager import BlockManagerOracle
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
        assert m.allocate("r", 30)
        assert len(m.table("r")) == case["blocks"]
        st = m.stats()
        assert st["used"] == case["blocks"]
        last_fill = 30 - (case["blocks"] - 1) * bs
        assert last_fill == case["last_block_tokens"]
        assert st["utilization"] == pytest.approx(30 / (case["blocks"] * bs))


def pin_short_queue_takes_nothing(cls):
    """ch. 12, 2.3: allocate answers False when the free queue cannot cover
    ceil(num_tokens / bs) blocks, and takes nothing."""
    m = cls(4, 16)
    assert m.allocate("a", 40)              # 3 blocks
    before = list(m.free_ids)
    assert not m.can_allocate(17)           # needs 2, 1 free
    assert m.allocate("b", 17) is False
    assert list(m.free_ids) == before and "b" not in m.seqs
    assert m.allocate("c", 16)              # exactly 1 block fits


def pin_fifo_order(cls):
    """ch. 12, 2.3 and 4.2: blocks come from the left of a FIFO queue in
    order; freed blocks join it at the right."""
    m = cls(8, 16)
    assert m.allocate("a", 40)
    assert m.table("a") == [0, 1, 2]
    assert m.allocate("b", 20)
    assert m.table("b") == [3, 4]
    m.free("a")
    assert list(m.free_ids) == [5, 6, 7, 0, 1, 2]
    assert m.allocate("c", 64)
    assert m.table("c") == [5, 6, 7, 0]


def pin_ref_count_release(cls):
    """ch. 12, 2.4: a block shared by two holders goes back to the free
    queue only when the last holder leaves."""
    m = cls(8, 16)
    assert m.allocate("a", 48)
    m.share("a", "b", 2)
    assert m.ref_count[:3] == [2, 2, 1]
    m.free("a")
    assert 0 not in m.free_ids and 1 not in m.free_ids and 2 in m.free_ids
    m.free("b")
    assert 0 in m.free_ids and 1 in m.free_ids
    assert all(r == 0 for r in m.ref_count)


def pin_release_order(cls):
    """ch. 12, 7 (exercise): two requests holding a ref_count-2 block finish
    in either order -- the final state (free set, reference counts) is the
    same; only the queue order of the freed blocks differs."""
    def run(order):
        m = cls(8, 16)
        assert m.allocate("a", 48)
        m.share("a", "b", 2)
        assert m.append_slot("b") is not None    # b's own block
        for s in order:
            m.free(s)
        return m

    x, y = run(["a", "b"]), run(["b", "a"])
    assert sorted(x.free_ids) == sorted(y.free_ids) == list(range(8))
    assert x.ref_count == y.ref_count
    assert x.used() == y.used() == 0


def pin_append_slot(cls):
    """vLLM source notes 2.1: the decode append takes the next slot of the
    last block when it has room, a new block when it is full; the slot is
    the one of the slot formula (pinned separately) at the new position."""
    m = cls(16, 16)
    assert m.allocate("a", 14, offset=1)          # flat positions 1..14
    s = m.append_slot("a")                        # position 15: same block
    assert s == m.table("a")[0] * 16 + 15 and len(m.table("a")) == 1
    s = m.append_slot("a")                        # position 16: new block
    assert len(m.table("a")) == 2 and s == m.table("a")[1] * 16
    # against the slot formula of the C oracle
    bt = np.array([m.table("a") + [-1] * 4], dtype=np.int32)
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
                assert m.allocate("a", n, offset=off)
                cap = m.capacity("a")
                assert cap == len(m.table("a")) * bs - off
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
