"""Parity of paged prefill / append attention (HIP, through the C ABI) with
the CPU oracle.

Each sequence's last n tokens are queries; query i sits at logical position
L - n + i and attends causally to tokens 0 .. L - n + i of its sequence, read
in place through the block table and its first-block offset.  Bar: max abs
error 2e-2 for bf16 inputs and 1e-5 for fp32 inputs against the float64
oracle; rows of queries that see no token are exactly zero.

Small cases run the oracle on the whole pool and span several 16-query
tiles, 16-position chunks, ragged tails and random offsets.  The full-size
case (the prefix-sharing batch, every suffix token a query) checks sampled
rows: a query at position P is the oracle's one-query prefill of the first
P + 1 tokens.
"""
import numpy as np
import pytest
import torch

import oracle as O
from paged_attention_decode_scatter_amd import native as N
from paged_attention_decode_scatter_amd import workloads as W
from tests.pkv_testlib import TOL, compact, host, max_abs_err, oracle_threads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.load_library()
    return torch.device("cuda:0")


def small(dev, dtype=torch.bfloat16, head_dim=128, group=4, num_kv_heads=2, seed=70,
          num_seqs=5, min_len=1, max_len=300, offsets="random", block_size=16,
          num_blocks=None):
    nb = num_blocks or (num_seqs * (max_len + 2 * block_size)) // block_size + 64
    return W.decode_batch(device=dev, seed=seed, num_seqs=num_seqs, min_len=min_len,
                          max_len=max_len, num_blocks=nb, num_layers=3,
                          num_kv_heads=num_kv_heads, head_dim=head_dim,
                          num_q_heads=num_kv_heads * group, dtype=dtype, layer=1,
                          offsets=offsets, block_size=block_size)


def queries(w, counts, seed):
    """q rows for `counts` queries per sequence, and q_start (int32, device)."""
    counts = [int(c) for c in counts]
    q_start = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    q = torch.empty((int(q_start[-1]), w.num_q_heads, w.head_dim), dtype=w.dtype,
                    device=w.k_pool.device)
    W.fill_normal_(q, seed)
    return q, torch.from_numpy(q_start).to(w.k_pool.device)


def run(w, q, q_start, max_q_len=None):
    """Prefill through the C ABI into an output prefilled with NaN, so any
    element the kernels fail to write shows up."""
    counts = (q_start[1:] - q_start[:-1]).cpu()
    mq = int(counts.max()) if max_q_len is None else max_q_len
    out = torch.full_like(q, float("nan"))
    return N.paged_attn_prefill(w.k_pool, w.v_pool, w.layer, q, q_start, w.block_tables,
                                w.seq_lens, w.offsets, mq, w.scale, out=out)


def oracle_for(w, q, q_start):
    k_c, v_c, bt_c, _ = compact(w.k_pool, w.v_pool, w.layer, w.block_tables)
    return O.prefill(k_c, v_c, 0, host(q), host(q_start), bt_c, host(w.seq_lens),
                     host(w.offsets), w.scale, num_threads=oracle_threads())


def random_counts(w, seed, lo=1):
    rng = np.random.default_rng(seed)
    lens = host(w.seq_lens)
    return [int(rng.integers(min(lo, l), l + 1)) if l > 0 else 0 for l in lens]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_prefill_small_grid(dev, dtype, head_dim, group):
    """Random n per sequence (1 .. L): several query tiles and ragged ones."""
    w = small(dev, dtype=dtype, head_dim=head_dim, group=group, seed=70 + group)
    q, qs = queries(w, random_counts(w, 170 + group), 270 + group)
    got = run(w, q, qs)
    ref = oracle_for(w, q, qs)
    assert max_abs_err(got, ref) <= TOL[dtype]


@pytest.mark.parametrize("group,head_dim", [(1, 128), (1, 64), (2, 128), (8, 64)])
def test_prefill_spans_several_workgroup_tiles(dev, group, head_dim):
    """Long query runs: several workgroup tiles per sequence (up to 384
    queries each for G = 1), ragged last tiles and wavefront groups with no
    query left."""
    w = small(dev, head_dim=head_dim, group=group, seed=150 + group, num_seqs=3, min_len=900,
              max_len=1300)
    lens = host(w.seq_lens)
    q, qs = queries(w, [int(lens[0]), 800, 397], 250 + group)
    got = run(w, q, qs)
    assert max_abs_err(got, oracle_for(w, q, qs)) <= TOL[w.dtype]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_whole_prompt(dev, dtype):
    """n = L: the whole prompt is new (plain causal attention); the first
    query sees only its own token, so its row is that token's V row."""
    w = small(dev, dtype=dtype, seed=80, num_seqs=4, min_len=1, max_len=200)
    lens = host(w.seq_lens)
    q, qs = queries(w, lens, 180)
    got = run(w, q, qs)
    ref = oracle_for(w, q, qs)
    assert max_abs_err(got, ref) <= TOL[dtype]


@pytest.mark.parametrize("bs", [1, 4, 32])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_other_block_sizes(dev, bs, dtype):
    """block_size below 16 (a chunk spans several blocks) and above it."""
    w = small(dev, dtype=dtype, seed=90 + bs, block_size=bs, max_len=260)
    q, qs = queries(w, random_counts(w, 190 + bs), 290 + bs)
    got = run(w, q, qs)
    assert max_abs_err(got, oracle_for(w, q, qs)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_edge_lengths_offsets_and_empty(dev, dtype):
    """Lengths around the 16-position chunk and 16-query tile, offsets 0, 1
    and 15, sequences with no queries, and an empty sequence."""
    w = small(dev, dtype=dtype, seed=100, num_seqs=12, min_len=64, max_len=64, offsets=None)
    lens = [1, 15, 16, 17, 33, 40, 0, 16, 17, 32, 33, 5]
    offs = [0, 1, 15, 0, 1, 15, 3, 15, 0, 1, 15, 2]
    counts = [1, 15, 16, 17, 16, 0, 0, 1, 17, 32, 20, 5]
    w.seq_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    w.offsets = torch.tensor(offs, dtype=torch.int32, device=dev)
    q, qs = queries(w, counts, 200)
    got = run(w, q, qs)
    assert max_abs_err(got, oracle_for(w, q, qs)) <= TOL[dtype]


def test_prefill_more_queries_than_tokens_gives_zero_rows(dev):
    """A query before the first token (position < 0) sees nothing: zeros."""
    w = small(dev, seed=110, num_seqs=3, min_len=20, max_len=20, offsets=None)
    w.seq_lens = torch.tensor([5, 20, 0], dtype=torch.int32, device=dev)
    q, qs = queries(w, [9, 20, 3], 210)   # 4 leading queries of seq 0 and all of seq 2 see nothing
    got = run(w, q, qs)
    ref = oracle_for(w, q, qs)
    assert max_abs_err(got, ref) <= TOL[w.dtype]
    assert torch.all(got[:4] == 0) and torch.all(got[-3:] == 0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_one_query_matches_decode(dev, dtype):
    """n = 1 is the decode step: both kernels meet the oracle's decode."""
    w = small(dev, dtype=dtype, seed=120, num_seqs=6, max_len=500)
    q, qs = queries(w, [1] * 6, 220)
    got = run(w, q, qs)
    k_c, v_c, bt_c, _ = compact(w.k_pool, w.v_pool, w.layer, w.block_tables)
    ref = O.decode(k_c, v_c, 0, host(q), bt_c, host(w.seq_lens), host(w.offsets), w.scale,
                   num_threads=oracle_threads())
    assert max_abs_err(got, ref) <= TOL[dtype]
    dec = N.paged_attn_decode(w.k_pool, w.v_pool, w.layer, q, w.block_tables, w.seq_lens,
                              w.offsets, w.max_seq_len, w.scale)
    assert max_abs_err(dec, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_ignores_unowned_nan_slots(dev, dtype):
    """Slots no sequence owns (before the offset, past the length) hold NaN
    and must not reach any output."""
    w = small(dev, dtype=dtype, seed=130, num_seqs=4, max_len=150)
    lens, offs, bt = host(w.seq_lens), host(w.offsets), host(w.block_tables)
    bs = w.block_size
    for s in range(w.num_seqs):
        for p in range(bt.shape[1] * bs):
            b = int(bt[s, p // bs])
            if b >= 0 and not (offs[s] <= p < offs[s] + lens[s]):
                w.k_pool[b, w.layer, p % bs] = float("nan")
                w.v_pool[b, w.layer, p % bs] = float("nan")
    q, qs = queries(w, random_counts(w, 230), 330)
    got = run(w, q, qs)
    assert max_abs_err(got, oracle_for(w, q, qs)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("mq", [32, 20])
def test_prefill_rows_beyond_max_q_len_are_untouched(dev, dtype, mq):
    """max_q_len bounds the queries computed per sequence: rows of a
    sequence past it are left as they were (here NaN), the rest are
    computed (also when max_q_len is not a multiple of the query tile)."""
    w = small(dev, dtype=dtype, seed=140, num_seqs=2, min_len=100, max_len=100, offsets=None)
    q, qs = queries(w, [40, 10], 240)
    got = run(w, q, qs, max_q_len=mq)
    ref = oracle_for(w, q, qs)
    assert torch.all(torch.isnan(got[mq:40]))
    keep = torch.ones(50, dtype=torch.bool)
    keep[mq:40] = False
    assert max_abs_err(got[keep.to(dev)], ref[keep.numpy()]) <= TOL[dtype]


def test_prefill_prefix_sharing_full_size(dev):
    """Prefix-sharing batch at full size (64 sequences sharing 32 physical
    blocks at a common first-block offset, ref count 64): every suffix token
    is a query, attending causally to the shared prefix and its own tokens.
    Every query row of two whole sequences (the one of median query count
    and the one of smallest count) against the oracle's prefill of those
    sequences, and sampled rows of 12 others against its one-query prefill of
    the first P + 1 tokens."""
    w = W.prefix_sharing(device=dev)
    lens = host(w.seq_lens).astype(np.int64)
    prefix = int(w.meta["shared_blocks"]) * w.block_size
    counts = [max(1, int(l) - prefix) for l in lens]
    q, qs = queries(w, counts, 250)
    got = run(w, q, qs)
    assert torch.isfinite(got).all()
    qs_h = host(qs)
    order = np.argsort(np.array(counts), kind="stable")
    for s in (int(order[len(order) // 2]), int(order[0])):
        rows = torch.arange(int(qs_h[s]), int(qs_h[s + 1]), device=dev)
        k_c, v_c, bt_c, _ = compact(w.k_pool, w.v_pool, w.layer, w.block_tables[s:s + 1])
        ref = O.prefill(k_c, v_c, 0, host(q[rows]), np.array([0, counts[s]], np.int32), bt_c,
                        lens[s:s + 1].astype(np.int32), host(w.offsets[s:s + 1]), w.scale,
                        num_threads=oracle_threads())
        err = max_abs_err(got[rows], ref)
        print(f"prefix-sharing prefill, sequence {s}: {counts[s]} query rows, max abs err {err:.3e}")
        assert err <= TOL[w.dtype]
    rng = np.random.default_rng(251)
    qs_h = host(qs)
    picks = []
    for s in rng.choice(w.num_seqs, size=12, replace=False):
        n = counts[s]
        for i in {0, n - 1, int(rng.integers(0, n))}:
            picks.append((int(s), i))
    rows = [int(qs_h[s]) + i for s, i in picks]
    sel = torch.tensor([s for s, _ in picks], dtype=torch.int64, device=dev)
    k_c, v_c, bt_c, _ = compact(w.k_pool, w.v_pool, w.layer, w.block_tables[sel])
    pos = np.array([int(lens[s]) - counts[s] + i for s, i in picks], np.int32)
    ref = O.prefill(k_c, v_c, 0, host(q[torch.tensor(rows, device=dev)]),
                    np.arange(len(picks) + 1, dtype=np.int32), bt_c, pos + 1,
                    host(w.offsets[sel]), w.scale, num_threads=oracle_threads())
    assert max_abs_err(got[torch.tensor(rows, device=dev)], ref) <= TOL[w.dtype]
