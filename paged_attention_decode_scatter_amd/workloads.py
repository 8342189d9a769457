"""Seeded synthetic inputs for the paged KV-cache path.

This module only builds inputs: pools filled with N(0, 1) values, block
tables drawn from seeded permutations of the pool's block ids, sequence
lengths, first-block offsets, query vectors, new K/V rows and the
(sequence, position) of every new row.  It computes no slot, gather or
attention arithmetic; both the HIP path and the CPU oracle consume what it
returns.

Workload shapes follow the pages' setups: block_size 16, a 16384-block pool
(262144-token capacity, mini-runtime's default configuration), K and V held
as separate (num_blocks, num_layers, block_size, num_kv_heads, head_dim)
tensors.  The five presets are:

  tiny            1 seq x 30 tokens, fp32, 8-block 1-layer pool, 2 kv heads,
                  head_dim 64, 4 query heads (GQA 2), scale 1/sqrt(64)
  decode_batch    32 seqs, seq_len ~ U[128, 2048], 32-layer bf16 pool,
                  8 kv heads, head_dim 128, 32 query heads
  prefill         8 requests x 1024 rows, 10% padding rows, layer 17
  prefix_sharing  64 seqs sharing a 512-token prefix (32 physical blocks)
                  that starts at a nonzero first-block offset; suffix
                  ~ U[0, 3584]
  long_context    8 seqs x 32768 tokens over a random permutation of all
                  16384 blocks, 64 query heads (GQA 8)
"""
from dataclasses import dataclass, field
import math
from typing import Optional

import torch

BLOCK_SIZE = 16
POOL_BLOCKS = 16384


@dataclass
class PagedWorkload:
    name: str
    dtype: torch.dtype
    num_blocks: int
    num_layers: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    num_q_heads: int
    layer: int
    scale: float
    seed: int
    block_tables: torch.Tensor  # int32 (num_seqs, bt_stride), unused entries -1
    seq_lens: torch.Tensor      # int32 (num_seqs,)
    offsets: torch.Tensor       # int32 (num_seqs,)
    k_pool: Optional[torch.Tensor] = None
    v_pool: Optional[torch.Tensor] = None
    q: Optional[torch.Tensor] = None
    # new rows to scatter: token i belongs to sequence token_seq[i]
    # (-1 = padding row) at logical position token_pos[i]
    token_seq: Optional[torch.Tensor] = None
    token_pos: Optional[torch.Tensor] = None
    k_new: Optional[torch.Tensor] = None
    v_new: Optional[torch.Tensor] = None
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max().item()) if self.num_seqs else 0

    @property
    def row_bytes(self) -> int:
        return self.num_kv_heads * self.head_dim * torch.tensor([], dtype=self.dtype).element_size()


def _cpu_gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed)


def fill_normal_(t: torch.Tensor, seed: int, chunk: int = 1 << 27) -> torch.Tensor:
    """Fill t with N(0, 1) (drawn in float32, then cast) from a generator
    seeded with `seed` on t's device; chunked so huge pools need little
    scratch memory."""
    gen = torch.Generator(device=t.device).manual_seed(seed)
    flat = t.view(-1)
    n = flat.numel()
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        flat[i:i + m].copy_(torch.randn(m, generator=gen, device=t.device, dtype=torch.float32))
    return t


def new_pool(num_blocks, num_layers, block_size, num_kv_heads, head_dim, dtype, device, seed):
    t = torch.empty((num_blocks, num_layers, block_size, num_kv_heads, head_dim),
                    dtype=dtype, device=device)
    return fill_normal_(t, seed)


def int8_pool_tensors(num_blocks, num_layers, block_size, num_kv_heads, head_dim, device, seed,
                      amax=3.0, chunk=1 << 28):
    """Random stored contents of one tensor of a quantised pool: codes
    uniform in [-127, 127] (int8, the pool layout) and one float32 scale per
    (block, layer, kv head, slot) drawn as amax / 127 * U(0.5, 1.5), so the
    stored values spread over about +-1.5 amax.  Chunked like fill_normal_."""
    gen = torch.Generator(device=device).manual_seed(seed)
    codes = torch.empty((num_blocks, num_layers, block_size, num_kv_heads, head_dim),
                        dtype=torch.int8, device=device)
    flat = codes.view(-1)
    for i in range(0, flat.numel(), chunk):
        m = min(chunk, flat.numel() - i)
        flat[i:i + m].copy_(torch.randint(-127, 128, (m,), generator=gen, device=device,
                                          dtype=torch.int32))
    u = torch.rand((num_blocks, num_layers, num_kv_heads, block_size), generator=gen,
                   device=device, dtype=torch.float32)
    scales = (u + 0.5) * (amax / 127.0)
    return codes, scales


def int4_pool_tensors(num_blocks, num_layers, block_size, num_kv_heads, head_dim, device, seed,
                      amax=3.0, chunk=1 << 28):
    """Random stored contents of one tensor of an int4 pool: uniformly
    random bytes (uint8, the pool layout with head_dim / 2 bytes per head
    row; every byte value, so every pair of four-bit codes, -8 included)
    and one float32 scale per (block, layer, kv head, slot) drawn as
    amax / 7 * U(0.5, 1.5).  Chunked like fill_normal_."""
    gen = torch.Generator(device=device).manual_seed(seed)
    codes = torch.empty((num_blocks, num_layers, block_size, num_kv_heads, head_dim // 2),
                        dtype=torch.uint8, device=device)
    flat = codes.view(-1)
    for i in range(0, flat.numel(), chunk):
        m = min(chunk, flat.numel() - i)
        flat[i:i + m].copy_(torch.randint(0, 256, (m,), generator=gen, device=device,
                                          dtype=torch.int32))
    u = torch.rand((num_blocks, num_layers, num_kv_heads, block_size), generator=gen,
                   device=device, dtype=torch.float32)
    scales = (u + 0.5) * (amax / 7.0)
    return codes, scales


def _tables_from_counts(counts, perm, stride=None):
    """Consecutive slices of `perm` as block tables, padded with -1."""
    stride = stride or max(1, max(counts) if counts else 1)
    bt = torch.full((len(counts), stride), -1, dtype=torch.int32)
    at = 0
    for i, c in enumerate(counts):
        bt[i, :c] = perm[at:at + c]
        at += c
    if at > perm.numel():
        raise ValueError("pool too small for the requested tables")
    return bt


def _n_blocks(tokens_with_offset: int, block_size: int) -> int:
    # table length needed to cover flat positions [0, tokens_with_offset)
    return -(-tokens_with_offset // block_size)


def _attach(w: PagedWorkload, device, with_pools=True, with_q=True):
    w.block_tables = w.block_tables.to(device)
    w.seq_lens = w.seq_lens.to(device)
    w.offsets = w.offsets.to(device)
    if with_pools:
        w.k_pool = new_pool(w.num_blocks, w.num_layers, w.block_size, w.num_kv_heads,
                            w.head_dim, w.dtype, device, w.seed * 16 + 1)
        w.v_pool = new_pool(w.num_blocks, w.num_layers, w.block_size, w.num_kv_heads,
                            w.head_dim, w.dtype, device, w.seed * 16 + 2)
    if with_q:
        w.q = fill_normal_(torch.empty((w.num_seqs, w.num_q_heads, w.head_dim),
                                       dtype=w.dtype, device=device), w.seed * 16 + 3)
    return w


def _new_rows(w: PagedWorkload, n: int, device):
    shape = (n, w.num_kv_heads, w.head_dim)
    w.k_new = fill_normal_(torch.empty(shape, dtype=w.dtype, device=device), w.seed * 16 + 4)
    w.v_new = fill_normal_(torch.empty(shape, dtype=w.dtype, device=device), w.seed * 16 + 5)


# --------------------------------------------------------------------------
# presets (keyword overrides shrink them for CPU-side tests)
# --------------------------------------------------------------------------
def tiny(device="cpu", seed=1000, **kw) -> PagedWorkload:
    nb = kw.get("num_blocks", 8)
    bs = kw.get("block_size", BLOCK_SIZE)
    L = kw.get("seq_len", 30)
    g = _cpu_gen(seed)
    perm = torch.randperm(nb, generator=g).to(torch.int32)
    nblk = _n_blocks(L, bs)
    w = PagedWorkload(
        name="tiny", dtype=kw.get("dtype", torch.float32), num_blocks=nb, num_layers=1,
        block_size=bs, num_kv_heads=2, head_dim=64, num_q_heads=4, layer=0,
        scale=1.0 / math.sqrt(64), seed=seed,
        block_tables=_tables_from_counts([nblk], perm),
        seq_lens=torch.tensor([L], dtype=torch.int32),
        offsets=torch.zeros(1, dtype=torch.int32))
    _attach(w, device)
    w.token_seq = torch.zeros(L, dtype=torch.int32, device=device)
    w.token_pos = torch.arange(L, dtype=torch.int32, device=device)
    _new_rows(w, L, device)
    return w


def decode_batch(device="cpu", seed=1001, num_seqs=32, min_len=128, max_len=2048,
                 num_blocks=POOL_BLOCKS, num_layers=32, num_kv_heads=8, head_dim=128,
                 num_q_heads=32, dtype=torch.bfloat16, layer=0, with_pools=True,
                 offsets=None, block_size=BLOCK_SIZE) -> PagedWorkload:
    g = _cpu_gen(seed)
    lens = torch.randint(min_len, max_len + 1, (num_seqs,), generator=g, dtype=torch.int64)
    if offsets is None:
        offs = torch.zeros(num_seqs, dtype=torch.int64)
    elif offsets == "random":
        offs = torch.randint(0, block_size, (num_seqs,), generator=g, dtype=torch.int64)
    else:
        offs = torch.as_tensor(offsets, dtype=torch.int64)
    perm = torch.randperm(num_blocks, generator=g).to(torch.int32)
    counts = [_n_blocks(int(l) + int(o), block_size) for l, o in zip(lens, offs)]
    w = PagedWorkload(
        name="decode_batch", dtype=dtype, num_blocks=num_blocks, num_layers=num_layers,
        block_size=block_size, num_kv_heads=num_kv_heads, head_dim=head_dim,
        num_q_heads=num_q_heads, layer=layer, scale=1.0 / math.sqrt(head_dim), seed=seed,
        block_tables=_tables_from_counts(counts, perm),
        seq_lens=lens.to(torch.int32), offsets=offs.to(torch.int32))
    return _attach(w, device, with_pools=with_pools)


def prefill(device="cpu", seed=1002, num_requests=8, prompt_len=1024, pad_fraction=0.10,
            random_padding=False, num_blocks=POOL_BLOCKS, num_layers=32, num_kv_heads=8,
            head_dim=128, dtype=torch.bfloat16, layer=17, with_pools=True) -> PagedWorkload:
    """num_requests x prompt_len rows; round(pad_fraction * rows) of them are
    padding.  Tail padding (default): each request's last rows are padding,
    so its first L_r rows are tokens 0..L_r-1.  random_padding: padding rows
    are drawn uniformly; every other row r of a request is token r."""
    g = _cpu_gen(seed)
    rows = num_requests * prompt_len
    n_pad = int(round(pad_fraction * rows))
    blocks_per_req = _n_blocks(prompt_len, BLOCK_SIZE)
    perm = torch.randperm(num_blocks, generator=g).to(torch.int32)
    bt = _tables_from_counts([blocks_per_req] * num_requests, perm)
    token_seq = torch.arange(num_requests, dtype=torch.int32).repeat_interleave(prompt_len)
    token_pos = torch.arange(prompt_len, dtype=torch.int32).repeat(num_requests)
    if random_padding:
        pad_rows = torch.randperm(rows, generator=g)[:n_pad]
        token_seq[pad_rows] = -1
        lens = torch.full((num_requests,), prompt_len, dtype=torch.int32)
    else:
        per = [n_pad // num_requests + (1 if r < n_pad % num_requests else 0)
               for r in range(num_requests)]
        lens = torch.tensor([prompt_len - p for p in per], dtype=torch.int32)
        for r in range(num_requests):
            token_seq[r * prompt_len + int(lens[r]):(r + 1) * prompt_len] = -1
    w = PagedWorkload(
        name="prefill" + ("_randpad" if random_padding else ""), dtype=dtype,
        num_blocks=num_blocks, num_layers=num_layers, block_size=BLOCK_SIZE,
        num_kv_heads=num_kv_heads, head_dim=head_dim, num_q_heads=num_kv_heads,
        layer=layer, scale=1.0 / math.sqrt(head_dim), seed=seed, block_tables=bt,
        seq_lens=lens, offsets=torch.zeros(num_requests, dtype=torch.int32))
    _attach(w, device, with_pools=with_pools, with_q=False)
    w.token_seq = token_seq.to(device)
    w.token_pos = token_pos.to(device)
    _new_rows(w, rows, device)
    w.meta["padding_rows"] = n_pad
    return w


def prefix_sharing(device="cpu", seed=1003, num_seqs=64, prefix_len=512, max_suffix=3584,
                   num_blocks=POOL_BLOCKS, num_layers=32, num_kv_heads=8, head_dim=128,
                   num_q_heads=32, dtype=torch.bfloat16, layer=0, with_pools=True,
                   offset=None) -> PagedWorkload:
    """All sequences start at the same nonzero first-block offset o and share
    the physical blocks that hold flat positions [0, prefix_len) of their
    tables (ref_count = num_seqs).  Every sequence then has private blocks:
    the first holds the prefix's last o tokens followed by its own suffix.
    seq_len = prefix_len + suffix, suffix ~ U[0, max_suffix]."""
    g = _cpu_gen(seed)
    o = int(torch.randint(1, BLOCK_SIZE, (1,), generator=g)) if offset is None else int(offset)
    shared = prefix_len // BLOCK_SIZE
    suffix = torch.randint(0, max_suffix + 1, (num_seqs,), generator=g, dtype=torch.int64)
    lens = prefix_len + suffix
    perm = torch.randperm(num_blocks, generator=g).to(torch.int32)
    shared_ids = perm[:shared]
    rest = perm[shared:]
    counts = [_n_blocks(int(l) + o, BLOCK_SIZE) for l in lens]
    stride = max(counts)
    bt = torch.full((num_seqs, stride), -1, dtype=torch.int32)
    at = 0
    for i, c in enumerate(counts):
        bt[i, :shared] = shared_ids
        bt[i, shared:c] = rest[at:at + c - shared]
        at += c - shared
    w = PagedWorkload(
        name="prefix_sharing", dtype=dtype, num_blocks=num_blocks, num_layers=num_layers,
        block_size=BLOCK_SIZE, num_kv_heads=num_kv_heads, head_dim=head_dim,
        num_q_heads=num_q_heads, layer=layer, scale=1.0 / math.sqrt(head_dim), seed=seed,
        block_tables=bt, seq_lens=lens.to(torch.int32),
        offsets=torch.full((num_seqs,), o, dtype=torch.int32))
    w.meta["shared_blocks"] = shared
    w.meta["ref_count"] = num_seqs
    w.meta["private_blocks"] = at
    return _attach(w, device, with_pools=with_pools)


def long_context(device="cpu", seed=1004, num_seqs=8, seq_len=32768, num_blocks=POOL_BLOCKS,
                 num_layers=32, num_kv_heads=8, head_dim=128, num_q_heads=64,
                 dtype=torch.bfloat16, layer=0, with_pools=True) -> PagedWorkload:
    g = _cpu_gen(seed)
    per = _n_blocks(seq_len, BLOCK_SIZE)
    perm = torch.randperm(num_blocks, generator=g).to(torch.int32)
    w = PagedWorkload(
        name="long_context", dtype=dtype, num_blocks=num_blocks, num_layers=num_layers,
        block_size=BLOCK_SIZE, num_kv_heads=num_kv_heads, head_dim=head_dim,
        num_q_heads=num_q_heads, layer=layer, scale=1.0 / math.sqrt(head_dim), seed=seed,
        block_tables=_tables_from_counts([per] * num_seqs, perm),
        seq_lens=torch.full((num_seqs,), seq_len, dtype=torch.int32),
        offsets=torch.zeros(num_seqs, dtype=torch.int32))
    return _attach(w, device, with_pools=with_pools)


def decode_tokens(w: PagedWorkload, device=None):
    """One new token per sequence at its last position (the decode step's
    write): token_seq = s, token_pos = seq_len[s] - 1, for seqs with
    seq_len > 0."""
    device = device or w.seq_lens.device
    lens = w.seq_lens.cpu()
    seqs = torch.nonzero(lens > 0).flatten().to(torch.int32)
    w.token_seq = seqs.to(device)
    w.token_pos = (lens[seqs.long()] - 1).to(torch.int32).to(device)
    _new_rows(w, int(seqs.numel()), device)
    return w


PRESETS = {
    "tiny": tiny,
    "decode_batch": decode_batch,
    "prefill": prefill,
    "prefix_sharing": prefix_sharing,
    "long_context": long_context,
}
