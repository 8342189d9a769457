"""Whole-block operations on the GPU, through the C ABI, against the oracle:
copy-on-write copies (kv_copy_blocks), swap out / in (kv_swap_out,
kv_swap_in), the combined (num_blocks, 2, layers, block_size, heads,
head_dim) layout, and copy-on-write end to end with the native block
manager.  Every byte comparison is bit-exact; decode outputs meet the
oracle's float64 decode within 2e-2 (bf16 inputs) or 1e-5 (fp32).
"""
import numpy as np
import pytest
import torch

import oracle as O
from paged_attention_decode_scatter_amd import native as N
from paged_attention_decode_scatter_amd import workloads as W
from tests.pkv_testlib import TOL, bits, host, max_abs_err, oracle_threads, row_starts

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.load_library()
    return torch.device("cuda:0")


def make_pools(dev, dtype, nb, nl, bs, h, d, combined, seed):
    """(k, v, keep): K and V pools filled with N(0, 1); with combined=True
    they are the two views of one (nb, 2, nl, bs, h, d) tensor `keep`."""
    if combined:
        kv = torch.empty((nb, 2, nl, bs, h, d), dtype=dtype, device=dev)
        W.fill_normal_(kv, seed)
        k, v = N.combined_views(kv)
        return k, v, kv
    k = torch.empty((nb, nl, bs, h, d), dtype=dtype, device=dev)
    v = torch.empty_like(k)
    W.fill_normal_(k, seed)
    W.fill_normal_(v, seed + 1)
    return k, v, None


def same_bits(t, a):
    return np.array_equal(bits(host(t)), bits(a))


def copy_pairs(nb, n, seed):
    """n valid pairs (distinct destinations, none of them a source) and
    three with an id outside the pool."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(nb)
    src = perm[:n].tolist() + [-1, 3, nb + 2]
    dst = perm[n:2 * n].tolist() + [5, nb, -7]
    return np.array(src, np.int32), np.array(dst, np.int32)


SHAPES = [
    # (dtype, layers, block_size, heads, head_dim): block bytes per tensor
    (torch.bfloat16, 3, 16, 2, 128),    # 24 KiB: one partial piece
    (torch.bfloat16, 5, 16, 8, 128),    # 160 KiB: 2.5 pieces of 64 KiB
    (torch.bfloat16, 32, 16, 8, 128),   # 1 MiB: the pool of the decode workloads
    (torch.float32, 3, 4, 2, 64),       # 6 KiB
]


@pytest.mark.parametrize("combined", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{str(s[0])[6:]}-L{s[1]}bs{s[2]}h{s[3]}d{s[4]}")
def test_copy_blocks_bit_exact(dev, shape, combined):
    dtype, nl, bs, h, d = shape
    nb = 24
    k, v, _ = make_pools(dev, dtype, nb, nl, bs, h, d, combined, seed=500 + nl)
    src, dst = copy_pairs(nb, 7, 501 + nl)
    k_ref, v_ref = host(k).copy(), host(v).copy()
    O.copy_blocks(k_ref, src, dst)
    O.copy_blocks(v_ref, src, dst)
    N.kv_copy_blocks(k, v, torch.from_numpy(src).to(dev), torch.from_numpy(dst).to(dev))
    torch.cuda.synchronize()
    assert same_bits(k, k_ref) and same_bits(v, v_ref)


def test_copy_blocks_k_only_and_empty(dev):
    """No V pool: K is copied, nothing else is touched; zero pairs enqueue
    nothing."""
    k, v, _ = make_pools(dev, torch.bfloat16, 16, 4, 16, 2, 128, False, seed=510)
    v0 = v.clone()
    src, dst = copy_pairs(16, 5, 511)
    k_ref = O.copy_blocks(host(k).copy(), src, dst)
    N.kv_copy_blocks(k, None, torch.from_numpy(src).to(dev), torch.from_numpy(dst).to(dev))
    empty = torch.empty(0, dtype=torch.int32, device=dev)
    N.kv_copy_blocks(k, v, empty, empty)
    torch.cuda.synchronize()
    assert same_bits(k, k_ref)
    assert torch.equal(v.view(torch.int16), v0.view(torch.int16))


@pytest.mark.parametrize("pin", [True, False])
@pytest.mark.parametrize("combined", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_swap_out_then_in(dev, dtype, combined, pin):
    """Swap out blocks given in an order with consecutive runs (one copy per
    run in a dense pool) and single ids; the host copy is the oracle's.
    Then swap them into other blocks: the pool is the oracle's swap_in."""
    nb = 30
    k, v, _ = make_pools(dev, dtype, nb, 3, 16, 2, 64, combined, seed=520)
    ids = np.array([3, 4, 5, 9, 2, 7, 8, 29, 0], np.int32)
    k_ref, v_ref = host(k).copy(), host(v).copy()
    kh, vh = N.kv_swap_out(k, v, ids, pin=pin)
    torch.cuda.synchronize()
    assert same_bits(kh, O.swap_out(k_ref, ids)) and same_bits(vh, O.swap_out(v_ref, ids))
    into = np.array([10, 11, 12, 13, 20, 1, 2, 3, 28], np.int32)
    N.kv_swap_in(k, v, into, kh, vh)
    torch.cuda.synchronize()
    O.swap_in(k_ref, into, O.swap_out(k_ref.copy(), ids))
    O.swap_in(v_ref, into, O.swap_out(v_ref.copy(), ids))
    assert same_bits(k, k_ref) and same_bits(v, v_ref)


def test_swap_k_only_and_bad_id(dev):
    k, v, _ = make_pools(dev, torch.bfloat16, 8, 2, 16, 2, 128, False, seed=530)
    kh, vh = N.kv_swap_out(k, None, [6, 1])
    torch.cuda.synchronize()
    assert vh is None and same_bits(kh, O.swap_out(host(k), [6, 1]))
    with pytest.raises(N.PagedKVError):
        N.kv_swap_out(k, v, [1, 8])
    with pytest.raises(N.PagedKVError):
        N.kv_swap_in(k, v, [-1], kh[:1], kh[:1])


def combined_copy(w):
    """The workload's pools copied into a combined cache; returns its K/V
    views and the cache."""
    nb, nl, bs, h, d = w.k_pool.shape
    kv = torch.empty((nb, 2, nl, bs, h, d), dtype=w.dtype, device=w.k_pool.device)
    kv[:, 0].copy_(w.k_pool)
    kv[:, 1].copy_(w.v_pool)
    k, v = N.combined_views(kv)
    return k, v, kv


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_combined_layout_matches_dense(dev, dtype):
    """Append, gather, decode (split and planned), the one-launch decode
    step and prefill on the combined layout: every output and every pool
    byte equals the same call's on separate dense K and V pools."""
    w = W.decode_batch(device=dev, seed=540, num_seqs=7, min_len=1, max_len=600,
                       num_blocks=7 * 632 // 16 + 64, num_layers=3, num_kv_heads=2, head_dim=128,
                       num_q_heads=8, dtype=dtype, layer=1, offsets="random")
    w = W.decode_tokens(w)
    k, v, kv = combined_copy(w)
    for kp, vp in ((w.k_pool, w.v_pool), (k, v)):
        N.kv_append(kp, vp, w.layer, w.k_new, w.v_new, w.block_tables, w.offsets, w.token_seq,
                    w.token_pos)
    torch.cuda.synchronize()
    assert torch.equal(k.contiguous(), w.k_pool) and torch.equal(v.contiguous(), w.v_pool)

    rows = int(w.seq_lens.sum())
    rs = row_starts(w.seq_lens)
    outs = []
    for kp, vp in ((w.k_pool, w.v_pool), (k, v)):
        ko = torch.full((rows, w.num_kv_heads, w.head_dim), float("nan"), dtype=dtype, device=dev)
        vo = torch.full_like(ko, float("nan"))
        N.kv_gather(kp, vp, w.layer, w.block_tables, w.seq_lens, w.offsets, rs, w.max_seq_len,
                    ko, vo)
        res = [ko, vo]
        splits = (0, 64, N.SPLIT_PLANNED) if dtype == torch.bfloat16 else (0, 64)
        for split in splits:
            res.append(N.paged_attn_decode(kp, vp, w.layer, w.q, w.block_tables, w.seq_lens,
                                           w.offsets, w.max_seq_len, w.scale,
                                           split_tokens=split))
        counts = [min(int(l), 20) for l in host(w.seq_lens)]
        qs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=dev)
        qp = torch.empty((int(qs[-1]), w.num_q_heads, w.head_dim), dtype=dtype, device=dev)
        W.fill_normal_(qp, 541)
        res.append(N.paged_attn_prefill(kp, vp, w.layer, qp, qs, w.block_tables, w.seq_lens,
                                        w.offsets, max(counts), w.scale))
        outs.append(res)
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))

    # the one-launch step on both layouts, starting from equal pools
    kn = torch.zeros((w.num_seqs, w.num_kv_heads, w.head_dim), dtype=dtype, device=dev)
    W.fill_normal_(kn, 542)
    vn = torch.zeros_like(kn)
    W.fill_normal_(vn, 543)
    steps = []
    for kp, vp in ((w.k_pool, w.v_pool), (k, v)):
        steps.append(N.paged_attn_decode_append(kp, vp, w.layer, w.q, kn, vn, w.block_tables,
                                                w.seq_lens, w.offsets, w.max_seq_len, w.scale))
    torch.cuda.synchronize()
    assert torch.equal(steps[0].view(torch.uint8), steps[1].view(torch.uint8))
    assert torch.equal(k.contiguous(), w.k_pool) and torch.equal(v.contiguous(), w.v_pool)
    ref = O.decode(host(w.k_pool), host(w.v_pool), w.layer, host(w.q), host(w.block_tables),
                   host(w.seq_lens), host(w.offsets), w.scale, num_threads=oracle_threads())
    assert max_abs_err(steps[1], ref) <= TOL[dtype]


@pytest.mark.parametrize("combined", [False, True])
def test_copy_on_write_end_to_end(dev, combined):
    """Sequence 1 holds a prompt of 40 tokens from first-block offset 3
    (blocks written with kv_append); sequence 2 shares all three blocks.
    Before sequence 1 writes token 40 into its shared last block, the
    manager gives it a fresh block (pkv_bm_cow) and kv_copy_blocks copies
    the contents; the token then lands in the copy.  Sequence 2 still reads
    the old block: its decode over the 40 prompt tokens is unchanged, and
    sequence 1's decode over 41 tokens meets the oracle.  A second write
    into the now private block needs no copy."""
    dtype, nb, nl, bs, h, d, layer = torch.bfloat16, 12, 2, 16, 2, 128, 1
    k, v, _ = make_pools(dev, dtype, nb, nl, bs, h, d, combined, seed=550)
    m = N.BlockManager(nb, bs)
    assert m.allocate(1, 40, offset=3)
    t1 = m.table(1)
    bt = torch.tensor([t1], dtype=torch.int32, device=dev)
    prompt_k = torch.empty((40, h, d), dtype=dtype, device=dev)
    prompt_v = torch.empty_like(prompt_k)
    W.fill_normal_(prompt_k, 551)
    W.fill_normal_(prompt_v, 552)
    zeros = torch.zeros(40, dtype=torch.int32, device=dev)
    N.kv_append(k, v, layer, prompt_k, prompt_v, bt, torch.tensor([3], dtype=torch.int32,
                device=dev), zeros, torch.arange(40, dtype=torch.int32, device=dev))
    m.share(1, 2, 3)
    assert m.ref_count[t1[2]] == 2

    k_ref, v_ref = host(k).copy(), host(v).copy()
    src, dst = m.cow(1, 2)
    assert src == t1[2] and dst != src and m.ref_count[src] == 1
    N.kv_copy_blocks(k, v, torch.tensor([src], dtype=torch.int32, device=dev),
                     torch.tensor([dst], dtype=torch.int32, device=dev))
    slot = m.append_slot(1)
    assert slot // bs == dst and slot % bs == (3 + 40) % bs
    new_k = torch.empty((1, h, d), dtype=dtype, device=dev)
    new_v = torch.empty_like(new_k)
    W.fill_normal_(new_k, 553)
    W.fill_normal_(new_v, 554)
    N.kv_scatter(k, v, layer, new_k, new_v, torch.tensor([slot], dtype=torch.int64, device=dev))
    # second token: the block is private now, written in place
    assert m.cow(1, 2) == (dst, dst)
    slot2 = m.append_slot(1)
    N.kv_scatter(k, v, layer, new_v, new_k, torch.tensor([slot2], dtype=torch.int64, device=dev))
    torch.cuda.synchronize()

    for pool, a, b in ((k_ref, new_k, new_v), (v_ref, new_v, new_k)):
        O.copy_blocks(pool, [src], [dst])
        O.scatter(pool, layer, host(a), np.array([slot], np.int64))
        O.scatter(pool, layer, host(b), np.array([slot2], np.int64))
    assert same_bits(k, k_ref) and same_bits(v, v_ref)

    tabs, _, offs = m.tables([1, 2])
    assert list(offs) == [3, 3] and tabs[0, 2] == dst and tabs[1, 2] == src
    q = torch.empty((2, 4 * h, d), dtype=dtype, device=dev)
    W.fill_normal_(q, 555)
    lens = np.array([42, 40], np.int32)
    scale = 1.0 / d ** 0.5
    out = N.paged_attn_decode(k, v, layer, q, torch.from_numpy(tabs).to(dev),
                              torch.from_numpy(lens).to(dev), torch.from_numpy(offs).to(dev), 42,
                              scale)
    ref = O.decode(k_ref, v_ref, layer, host(q), tabs, lens, offs, scale)
    assert max_abs_err(out, ref) <= TOL[dtype]
    # sequence 2's 40 tokens are the prompt, read from the old block
    ref2 = O.decode(k_ref, v_ref, layer, host(q[1:]), tabs[:1], np.array([40], np.int32),
                    offs[:1], scale)
    assert max_abs_err(out[1:], ref2) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_read_blocks_checksum(dev, dtype):
    """kv_read_blocks (the read-rate reference the bench times) folds the
    layer slice of K and V of each listed block into the XOR of its 32-bit
    words: compared bit for bit with the same fold on the host; ids outside
    the pool give 0; V omitted reads K only."""
    g = torch.Generator().manual_seed(77)
    nb, nl, bs, h, d = 40, 3, 16, 4, 64
    k = torch.randn((nb, nl, bs, h, d), generator=g).to(dtype).to(dev)
    v = torch.randn((nb, nl, bs, h, d), generator=g).to(dtype).to(dev)
    ids = torch.tensor([3, 0, 39, -1, 17, 40, 3, 22], dtype=torch.int32, device=dev)
    layer = 2

    def fold(t, b):
        words = t[b, layer].contiguous().view(torch.int32).cpu().numpy().astype(np.uint32)
        return int(np.bitwise_xor.reduce(words.ravel()))

    got = N.kv_read_blocks(k, v, layer, ids).cpu().numpy().astype(np.uint32)
    got_k = N.kv_read_blocks(k, None, layer, ids).cpu().numpy().astype(np.uint32)
    for i, b in enumerate(ids.cpu().tolist()):
        if 0 <= b < nb:
            assert got[i] == fold(k, b) ^ fold(v, b), i
            assert got_k[i] == fold(k, b), i
        else:
            assert got[i] == 0 and got_k[i] == 0, i
