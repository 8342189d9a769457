"""CPU oracle of the host block manager -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline may use
this module; the library never does.

A plain Python statement of the allocator the pages describe:

  * "vLLM PagedAttention source notes", 2.1 Block Manager and Block Table:
    a global pool of fixed-size physical blocks; per-sequence block tables
    (logical block i -> physical id); allocate / free / append_slot /
    can_allocate; the decode append takes a free slot in the last block if
    it is not full, otherwise a new block.
  * mini-runtime ch. 12 "Paged KV Cache", 2.2 BlockTable: block ids in
    logical order, the first-block offset, capacity = blocks * bs - offset;
    2.3 KVCacheManager: per-block ref_count / is_free, a FIFO deque of free
    ids; allocate(num_tokens) needs ceil(num_tokens / bs) blocks, answers
    False when the free queue is short (nothing is taken then), otherwise
    pops that many from the left, in order, into the table; 2.4 ref_count:
    inc_ref adds a holder, dec_ref removes one and a block whose count
    reaches zero goes back to the free queue; 4.2: FIFO allocation.

Readings where the pages are silent (stated, not invented):
  * a block returned to the free queue goes to its right end (the deque's
    append), so FIFO means "least recently freed first";
  * free(seq) drops one reference from each block of the sequence's table,
    in table order;
  * append_slot counts capacity with the offset: a sequence of L tokens
    with offset o fills flat positions o .. o+L-1 of its table; the new
    token's slot is table[(o+L)//bs]*bs + (o+L)%bs;
  * share(src, dst, n): dst starts with src's first n blocks (one more
    reference each) and src's offset, holding the n*bs - offset tokens
    they can carry (whole-block sharing, as prefix sharing needs);
  * statistics: used = blocks not in the free queue; peak = the largest
    used count seen; utilisation = live tokens / (distinct used blocks *
    bs), live tokens counting each (block, slot) once;
  * cow(seq, j), the copy-on-write that "vLLM PagedAttention" sharing adds
    to ref_count (ch. 12, 3.1 industrial implementations, the sharing row):
    before a sequence writes into table entry j whose block other holders
    share (count > 1), it takes a new block from the free queue's front,
    the same FIFO take as allocate, puts it at entry j, and gives up one
    reference to the old block (which keeps its other holders); the caller
    copies the block's contents from old to new.  An unshared block needs
    no copy (the answer is (b, b), nothing changes); with an empty free
    queue the answer is False and nothing changes, as for allocate.

Parity unpinned: nothing (pins in tests/test_block_manager.py).
"""
from collections import deque
from math import ceil


class BlockManagerOracle:
    def __init__(self, num_blocks, block_size):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref_count = [0] * num_blocks
        self.free_ids = deque(range(num_blocks))
        self.seqs = {}          # seq id -> {"blocks": [...], "offset": o, "len": L}
        self.peak_used = 0

    # ---- queries -------------------------------------------------------
    def blocks_for(self, num_tokens, offset=0):
        return ceil((offset + num_tokens) / self.block_size) if num_tokens > 0 else 0

    def can_allocate(self, num_tokens, offset=0):
        return self.blocks_for(num_tokens, offset) <= len(self.free_ids)

    def used(self):
        return self.num_blocks - len(self.free_ids)

    def capacity(self, seq):
        st = self.seqs[seq]
        return len(st["blocks"]) * self.block_size - st["offset"]

    def _note_peak(self):
        self.peak_used = max(self.peak_used, self.used())

    # ---- allocation ----------------------------------------------------
    def allocate(self, seq, num_tokens, offset=0):
        """A new sequence of num_tokens tokens: True, or False with nothing
        taken when the free queue is short."""
        if seq in self.seqs:
            raise ValueError("sequence exists")
        if not 0 <= offset < self.block_size or num_tokens < 0:
            raise ValueError("bad offset or length")
        need = self.blocks_for(num_tokens, offset)
        if need > len(self.free_ids):
            return False
        blocks = []
        for _ in range(need):
            b = self.free_ids.popleft()
            self.ref_count[b] = 1
            blocks.append(b)
        self.seqs[seq] = {"blocks": blocks, "offset": offset, "len": num_tokens}
        self._note_peak()
        return True

    def share(self, src, dst, num_blocks):
        if dst in self.seqs:
            raise ValueError("sequence exists")
        s = self.seqs[src]
        if not 0 < num_blocks <= len(s["blocks"]):
            raise ValueError("bad block count")
        blocks = list(s["blocks"][:num_blocks])
        for b in blocks:
            self.ref_count[b] += 1
        self.seqs[dst] = {"blocks": blocks, "offset": s["offset"],
                          "len": num_blocks * self.block_size - s["offset"]}

    def append_slot(self, seq):
        """Slot of the sequence's next token, taking a new block when the
        last one is full; None (nothing changed) when none is free."""
        st = self.seqs[seq]
        p = st["offset"] + st["len"]
        j, s = divmod(p, self.block_size)
        if j == len(st["blocks"]):
            if not self.free_ids:
                return None
            b = self.free_ids.popleft()
            self.ref_count[b] = 1
            st["blocks"].append(b)
            self._note_peak()
        st["len"] += 1
        return st["blocks"][j] * self.block_size + s

    def cow(self, seq, index):
        """Copy-on-write of table entry `index` of `seq`: (old, new) block
        ids (old == new when the block is not shared), or False with
        nothing changed when a copy is needed and no block is free."""
        st = self.seqs[seq]
        if not 0 <= index < len(st["blocks"]):
            raise ValueError("bad table index")
        b = st["blocks"][index]
        if self.ref_count[b] <= 1:
            return (b, b)
        if not self.free_ids:
            return False
        nb = self.free_ids.popleft()
        self.ref_count[nb] = 1
        st["blocks"][index] = nb
        self.dec_ref(b)
        self._note_peak()
        return (b, nb)

    # ---- release ---------------------------------------------------------
    def inc_ref(self, block):
        if self.ref_count[block] <= 0:
            raise ValueError("block is free")
        self.ref_count[block] += 1

    def dec_ref(self, block):
        if self.ref_count[block] <= 0:
            raise ValueError("block is free")
        self.ref_count[block] -= 1
        if self.ref_count[block] == 0:
            self.free_ids.append(block)

    def free(self, seq):
        st = self.seqs.pop(seq)
        for b in st["blocks"]:
            self.dec_ref(b)

    # ---- export ----------------------------------------------------------
    def table(self, seq):
        return list(self.seqs[seq]["blocks"])

    def stats(self):
        live = set()
        for st in self.seqs.values():
            for t in range(st["len"]):
                p = st["offset"] + t
                live.add((st["blocks"][p // self.block_size], p % self.block_size))
        used_blocks = {b for b in range(self.num_blocks) if self.ref_count[b] > 0}
        util = len(live) / (len(used_blocks) * self.block_size) if used_blocks else 0.0
        return {"free": len(self.free_ids), "used": self.used(), "peak_used": self.peak_used,
                "live_tokens": len(live), "utilization": util}
