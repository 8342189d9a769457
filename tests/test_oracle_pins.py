"""Pins of the CPU oracle to what the pages fix (no GPU needed).

Each test ties an oracle function to something other than itself: a worked
example printed on the pages (tests/golden, each fixture citing its page), a
closed form, a second formulation taken from another passage of the pages,
or a library routine (torch's scaled_dot_product_attention in float64).

Sources:
  [P1] mini-vllm tutorial, "step14_2 - index_select gather"
  [P2] "vLLM PagedAttention source notes"
  [P3] mini-runtime, chapter 12 "Paged KV Cache"
"""
import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle as O
from tests.conftest import golden

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def tagged_pool(nb, nl, bs, h, d):
    """float32 pool whose every element encodes its own coordinates, so a
    gathered row tells exactly where it came from (all values < 2**24, so
    exact in float32)."""
    b, l, s, hh, dd = np.meshgrid(np.arange(nb), np.arange(nl), np.arange(bs),
                                  np.arange(h), np.arange(d), indexing="ij")
    code = ((((b * nl + l) * bs + s) * h + hh) * d + dd).astype(np.float32)
    assert code.max() < 2 ** 24
    return np.ascontiguousarray(code)


def untag(vals, nl, bs, h, d):
    code = vals.astype(np.int64)
    dd = code % d
    code //= d
    hh = code % h
    code //= h
    s = code % bs
    code //= bs
    l = code % nl
    b = code // nl
    return b, l, s, hh, dd


def random_bits_pool(rng, shape, dtype):
    """Random bit patterns (including NaN payloads) so byte-exact copies
    are checked, not value-equal ones."""
    if dtype == np.uint16:
        return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    return rng.integers(0, 1 << 32, size=shape, dtype=np.uint32).view(np.float32)


def as_bits(a):
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


# ---------------------------------------------------------------------------
# worked examples from the pages
# ---------------------------------------------------------------------------
def test_block_mapping_figure():
    """[P3 sec. 2.1 figure] tokens 0-15 -> block 7, 16-31 -> block 3,
    32-47 -> block 12; reading: token first+k of a range sits at slot k."""
    g = golden("p3_block_mapping.json")
    bs = g["block_size"]
    bt = np.array([g["block_table"]], dtype=np.int32)
    n = 48
    slots = O.slot_mapping(bt, [g["offset"]], np.zeros(n, np.int32),
                           np.arange(n, dtype=np.int32), bs)
    pool = tagged_pool(13, 1, bs, 1, 2)
    rows = O.gather(pool, 0, bt, np.array([n], np.int32), np.array([g["offset"]], np.int32))
    b, _, s, _, _ = untag(rows[:, 0, 0], 1, bs, 1, 2)
    for r in g["ranges"]:
        for t in range(r["first_token"], r["last_token"] + 1):
            assert slots[t] // bs == r["physical_block"]
            assert slots[t] % bs == t - r["first_token"]
            assert b[t] == r["physical_block"]
            assert s[t] == t - r["first_token"]


def test_think_question_30_tokens():
    """[P3 think questions] 30 tokens: 2 blocks / 32 slots at bs 16 (last
    block 14/16), 8 blocks / 32 slots at bs 4 (last block 2/4); [P2 sec. 3]
    fragmentation formula gives 2/32 in both cases."""
    g = golden("p3_think_30_tokens.json")
    n = g["num_tokens"]
    for c in g["cases"]:
        bs = c["block_size"]
        nblk = O.blocks_needed(n, bs)
        assert nblk == c["blocks"]
        assert nblk * bs == c["slots"]
        assert O.last_block_fill(n, bs) == c["last_block_tokens"]
        assert O.last_block_fill(n, bs) / bs == c["last_block_utilisation"]
        assert O.fragmentation_ratio(nblk, bs, n) == g["fragmentation_ratio_both"]
        # the gather walks exactly that many blocks and takes that many rows
        # from the last one
        pool = tagged_pool(nblk + 1, 1, bs, 1, 1)
        bt = np.arange(nblk, 0, -1, dtype=np.int32)[None, :]
        rows = O.gather(pool, 0, bt, np.array([n], np.int32), np.zeros(1, np.int32))
        b, _, _, _, _ = untag(rows[:, 0, 0], 1, bs, 1, 1)
        assert sorted(set(b.tolist())) == sorted(bt[0].tolist())
        assert int((b == bt[0, -1]).sum()) == c["last_block_tokens"]


def test_waste_example_arithmetic():
    """[P2 sec. 3] 128 requests x 8 wasted slots x 72 KB/token ~ 74 MB, and
    internal fragmentation comes only from each request's last block."""
    g = golden("p2_waste_example.json")
    waste = (g["requests"] * g["wasted_fraction_of_last_block"] * g["block_size"]
             * g["kv_bytes_per_token_kb"] * 1000)
    assert round(waste / 1e6) == g["stated_waste_mb"]
    # a request of 1 + 1/2 blocks wastes half a block
    assert O.fragmentation_ratio(2, 16, 24) == pytest.approx(8 / 32)


def test_fragmentation_below_bound_on_decode_batch_tables():
    """[P2 sec. 3] fragmentation < 4% when only last blocks are partial: the
    decode-batch tables (seq_len ~ U[128, 2048], bs 16) satisfy it."""
    from paged_attention_decode_scatter_amd import workloads

    w = workloads.decode_batch(with_pools=False, num_blocks=16384)
    lens = w.seq_lens.numpy().astype(np.int64)
    allocated = int((w.block_tables.numpy() >= 0).sum())
    assert allocated == sum(O.blocks_needed(int(l), 16) for l in lens)
    frag = O.fragmentation_ratio(allocated, 16, int(lens.sum()))
    assert 0 < frag < golden("p2_waste_example.json")["stated_fragmentation_bound"]


# ---------------------------------------------------------------------------
# capacity and the offset
# ---------------------------------------------------------------------------
@settings(max_examples=200, deadline=None)
@given(bs=st.sampled_from([1, 2, 4, 16]), nblk=st.integers(1, 5), data=st.data())
def test_gather_accepts_exactly_capacity(bs, nblk, data):
    """[P3 sec. 2.2] capacity = num_blocks*block_size - offset: the oracle's
    table walk reads seq_len = capacity and refuses capacity + 1."""
    off = data.draw(st.integers(0, bs - 1))
    cap = O.capacity(nblk, bs, off)
    pool = tagged_pool(nblk, 1, bs, 1, 1)
    bt = np.arange(nblk, dtype=np.int32)[None, :]
    rows = O.gather(pool, 0, bt, np.array([cap], np.int32), np.array([off], np.int32))
    assert rows.shape[0] == cap
    with pytest.raises(ValueError):
        O.gather(pool, 0, bt, np.array([cap + 1], np.int32), np.array([off], np.int32))


def test_offset_shifts_the_read():
    """[P3 sec. 2.2] ignoring the first-block offset misaligns the read: with
    offset o, logical token 0 is slot o of the first block."""
    bs = 16
    pool = tagged_pool(4, 1, bs, 1, 1)
    bt = np.array([[2, 0, 3]], np.int32)
    for o in range(bs):
        rows = O.gather(pool, 0, bt, np.array([20], np.int32), np.array([o], np.int32))
        b, _, s, _, _ = untag(rows[:, 0, 0], 1, bs, 1, 1)
        assert (b[0], s[0]) == (2, o)
        # the row after the first block's last slot is slot 0 of the second block
        k = bs - o
        assert (b[k], s[k]) == (0, 0)


# ---------------------------------------------------------------------------
# gather: loop-and-cat (C) against the flattened-index form and a Python loop
# ---------------------------------------------------------------------------
@settings(max_examples=300, deadline=None)
@given(bs=st.sampled_from([1, 2, 4, 16]), nb=st.integers(1, 6), h=st.integers(1, 3),
       d=st.sampled_from([1, 2, 8]), nl=st.integers(1, 3), bf16=st.booleans(),
       seed=st.integers(0, 2 ** 31 - 1), data=st.data())
def test_gather_formulations_agree(bs, nb, h, d, nl, bf16, seed, data):
    """[P1 "Problem"] loop-and-cat == [P1 "Solution"] flat advanced indexing,
    both with the [P3 sec. 2.2] offset, on random tiny pools, byte for byte."""
    rng = np.random.default_rng(seed)
    dt = np.uint16 if bf16 else np.float32
    pool = random_bits_pool(rng, (nb, nl, bs, h, d), dt)
    nt = data.draw(st.integers(1, nb))
    table = rng.permutation(nb)[:nt].astype(np.int32)
    off = data.draw(st.integers(0, bs - 1))
    L = data.draw(st.integers(0, O.capacity(nt, bs, off)))
    layer = data.draw(st.integers(0, nl - 1))
    got = O.gather(pool, layer, table[None, :], np.array([L], np.int32), np.array([off], np.int32))
    ref_flat = O.gather_flat_index(pool[:, layer], table, L, bs, off)
    ref_loop = O.gather_loop_cat(pool[:, layer], table.tolist(), L, bs, off)
    assert got.shape == (L, h, d)
    assert np.array_equal(as_bits(got), as_bits(ref_flat))
    assert np.array_equal(as_bits(got), as_bits(ref_loop))


def test_gather_multi_sequence_concatenates_in_order():
    rng = np.random.default_rng(7)
    bs, nb = 4, 12
    pool = random_bits_pool(rng, (nb, 2, bs, 2, 4), np.float32)
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((3, 5), -1, np.int32)
    bt[0, :3], bt[1, :4], bt[2, :2] = perm[:3], perm[3:7], perm[7:9]
    lens = np.array([9, 0, 7], np.int32)
    offs = np.array([2, 1, 1], np.int32)
    got = O.gather(pool, 1, bt, lens, offs)
    parts = [O.gather_flat_index(pool[:, 1], bt[i][bt[i] >= 0], int(lens[i]), bs, int(offs[i]))
             for i in range(3)]
    assert np.array_equal(as_bits(got), as_bits(np.concatenate(parts)))


# ---------------------------------------------------------------------------
# scatter
# ---------------------------------------------------------------------------
@settings(max_examples=200, deadline=None)
@given(bs=st.sampled_from([1, 2, 4, 16]), nb=st.integers(1, 6), nl=st.integers(1, 3),
       bf16=st.booleans(), seed=st.integers(0, 2 ** 31 - 1), data=st.data())
def test_scatter_matches_index_put_and_leaves_rest(bs, nb, nl, bf16, seed, data):
    """[P1 "relation to step14_1"] scatter == kv_pool[blocks, slots] = K with
    -1 rows dropped [P2 sec. 2.2]; every other byte of the pool unchanged."""
    rng = np.random.default_rng(seed)
    dt = np.uint16 if bf16 else np.float32
    h, d = 2, 4
    pool = random_bits_pool(rng, (nb, nl, bs, h, d), dt)
    before = pool.copy()
    n_slots = nb * bs
    n = data.draw(st.integers(0, n_slots + 3))
    uniq = rng.permutation(n_slots)[: min(n, n_slots)]
    slots = np.concatenate([uniq, -np.ones(n - uniq.size, np.int64)]).astype(np.int64)
    rng.shuffle(slots)
    layer = data.draw(st.integers(0, nl - 1))
    src = random_bits_pool(rng, (n, h, d), dt)
    got = O.scatter(pool.copy(), layer, src, slots)
    ref = before.copy()
    O.scatter_index_put(ref[:, layer], slots, src, bs)
    assert np.array_equal(as_bits(got), as_bits(ref))
    # untouched: other layers, and unwritten slots of this layer
    mask = np.ones((nb, nl, bs), bool)
    w = slots[slots >= 0]
    mask[w // bs, layer, w % bs] = False
    assert np.array_equal(as_bits(got)[mask], as_bits(before)[mask])


def test_scatter_refuses_out_of_pool_slots():
    pool = np.zeros((2, 1, 4, 1, 1), np.float32)
    with pytest.raises(ValueError):
        O.scatter(pool, 0, np.ones((1, 1, 1), np.float32), np.array([8], np.int64))
    with pytest.raises(ValueError):
        O.scatter(pool, 0, np.ones((1, 1, 1), np.float32), np.array([-2], np.int64))


@settings(max_examples=150, deadline=None)
@given(bs=st.sampled_from([1, 2, 4, 16]), seed=st.integers(0, 2 ** 31 - 1), data=st.data())
def test_gather_of_scatter_is_identity(bs, seed, data):
    """[P1 "relation to step14_1"] write and read use the same index math, so
    gather(scatter(K)) == K.  Slots come from the slot formula [P2 sec. 2.2]
    with the first-block offset [P3 sec. 2.2]; padding rows are skipped."""
    rng = np.random.default_rng(seed)
    nseq = data.draw(st.integers(1, 4))
    offs = np.array([data.draw(st.integers(0, bs - 1)) for _ in range(nseq)], np.int32)
    lens = np.array([data.draw(st.integers(0, 3 * bs)) for _ in range(nseq)], np.int32)
    counts = [O.blocks_needed(int(l) + int(o), bs) for l, o in zip(lens, offs)]
    nb = sum(counts) + 2
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((nseq, max(max(counts), 1)), -1, np.int32)
    at = 0
    for i, c in enumerate(counts):
        bt[i, :c] = perm[at:at + c]
        at += c
    tseq = np.concatenate([np.full(l, i, np.int32) for i, l in enumerate(lens)] + [np.full(3, -1, np.int32)])
    tpos = np.concatenate([np.arange(l, dtype=np.int32) for l in lens] + [np.zeros(3, np.int32)])
    order = rng.permutation(tseq.size)
    tseq, tpos = tseq[order], tpos[order]
    slots = O.slot_mapping(bt, offs, tseq, tpos, bs)
    assert np.array_equal(slots < 0, tseq < 0)
    h, d, nl, layer = 2, 3, 2, 1
    pool = random_bits_pool(rng, (nb, nl, bs, h, d), np.float32)
    rows = random_bits_pool(rng, (tseq.size, h, d), np.float32)
    O.scatter(pool, layer, rows, slots)
    got = O.gather(pool, layer, bt, lens, offs)
    # expected: for each sequence, its rows in logical-position order
    want = []
    for i in range(nseq):
        idx = np.nonzero(tseq == i)[0]
        idx = idx[np.argsort(tpos[idx])]
        want.append(rows[idx])
    want = np.concatenate(want) if want else rows[:0]
    assert np.array_equal(as_bits(got), as_bits(want))
    # and the flat-index gather of [P1 "Solution"] reads the same rows back
    for i in range(nseq):
        if lens[i]:
            flat = O.gather_flat_index(pool[:, layer], bt[i], int(lens[i]), bs, int(offs[i]))
            idx = np.nonzero(tseq == i)[0]
            idx = idx[np.argsort(tpos[idx])]
            assert np.array_equal(as_bits(flat), as_bits(rows[idx]))


def test_slot_mapping_refuses_positions_past_the_table():
    bt = np.array([[3, 1]], np.int32)
    with pytest.raises(ValueError):
        O.slot_mapping(bt, [4], np.zeros(1, np.int32), np.array([28], np.int32), 16)
    # position 27 with offset 4 is flat 31: the last slot of the table
    s = O.slot_mapping(bt, [4], np.zeros(1, np.int32), np.array([27], np.int32), 16)
    assert s[0] // 16 == 1 and s[0] % 16 == 15


# ---------------------------------------------------------------------------
# decode attention
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x):
    """Round-to-nearest-even float32 -> bf16 bit patterns (test input prep)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(a):
    return bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def make_decode_case(rng, nseq, hkv, G, d, bs, bf16, max_len=40, nl=2, offsets=True):
    lens = rng.integers(1, max_len + 1, size=nseq).astype(np.int32)
    offs = (rng.integers(0, bs, size=nseq) if offsets else np.zeros(nseq, np.int64)).astype(np.int32)
    counts = [O.blocks_needed(int(l) + int(o), bs) for l, o in zip(lens, offs)]
    nb = sum(counts) + 3
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((nseq, max(counts)), -1, np.int32)
    at = 0
    for i, c in enumerate(counts):
        bt[i, :c] = perm[at:at + c]
        at += c
    shape = (nb, nl, bs, hkv, d)
    kf = rng.standard_normal(shape).astype(np.float32)
    vf = rng.standard_normal(shape).astype(np.float32)
    qf = rng.standard_normal((nseq, hkv * G, d)).astype(np.float32)
    if bf16:
        return (f32_to_bf16_bits(kf), f32_to_bf16_bits(vf), f32_to_bf16_bits(qf), bt, lens, offs)
    return kf, vf, qf, bt, lens, offs


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_decode_matches_torch_sdpa(bf16, G):
    """[P2 sec. 2.3; P3 sec. 3.1] decode = gather then standard attention:
    compared with torch's scaled_dot_product_attention in float64 on K/V
    gathered by the flat-index form [P1 "Solution"], kv heads repeated per
    contiguous group of G query heads."""
    rng = np.random.default_rng(100 + G + 10 * bf16)
    hkv, d, bs, layer = 2, 16, 4, 1
    k, v, q, bt, lens, offs = make_decode_case(rng, 5, hkv, G, d, bs, bf16)
    scale = 0.3
    got = O.decode(k, v, layer, q, bt, lens, offs, scale, num_threads=3)
    for s in range(len(lens)):
        kc = to_f64(O.gather_flat_index(k[:, layer], bt[s], int(lens[s]), bs, int(offs[s])))
        vc = to_f64(O.gather_flat_index(v[:, layer], bt[s], int(lens[s]), bs, int(offs[s])))
        K = torch.from_numpy(kc).permute(1, 0, 2).repeat_interleave(G, dim=0)  # (Hq, L, D)
        V = torch.from_numpy(vc).permute(1, 0, 2).repeat_interleave(G, dim=0)
        Q = torch.from_numpy(to_f64(q[s]))[:, None, :]                          # (Hq, 1, D)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[:, 0]
        np.testing.assert_allclose(got[s], ref.numpy(), rtol=0, atol=1e-12)


def test_decode_single_token_returns_v():
    """softmax over one score is 1: out = V[token 0] exactly."""
    rng = np.random.default_rng(3)
    k, v, q, bt, lens, offs = make_decode_case(rng, 3, 2, 2, 8, 4, True)
    lens[:] = 1
    got = O.decode(k, v, 0, q, bt, lens, offs, 0.5)
    for s in range(3):
        row = v[bt[s, 0], 0, offs[s]]  # (hkv, d)
        for h in range(4):
            assert np.array_equal(got[s, h], bf16_bits_to_f64(row[h // 2]))


@pytest.mark.parametrize("mode", ["zero_q", "zero_scale"])
def test_decode_uniform_weights_give_mean(mode):
    """all scores equal (q = 0 or scale = 0) -> out is the plain mean of V."""
    rng = np.random.default_rng(5)
    bs, layer = 4, 1
    k, v, q, bt, lens, offs = make_decode_case(rng, 4, 2, 2, 8, bs, False)
    scale = 0.7
    if mode == "zero_q":
        q[:] = 0
    else:
        scale = 0.0
    got = O.decode(k, v, layer, q, bt, lens, offs, scale)
    for s in range(4):
        vc = O.gather_flat_index(v[:, layer], bt[s], int(lens[s]), bs, int(offs[s])).astype(np.float64)
        for h in range(4):
            np.testing.assert_allclose(got[s, h], vc[:, h // 2].mean(axis=0), rtol=0, atol=1e-13)


def test_decode_constant_v():
    rng = np.random.default_rng(6)
    k, v, q, bt, lens, offs = make_decode_case(rng, 3, 1, 4, 8, 4, False)
    v[:] = np.float32(1.25)
    got = O.decode(k, v, 0, q, bt, lens, offs, 1.0)
    np.testing.assert_allclose(got, 1.25, rtol=1e-15, atol=0)


def test_decode_empty_sequence_is_zero():
    rng = np.random.default_rng(8)
    k, v, q, bt, lens, offs = make_decode_case(rng, 3, 2, 2, 8, 4, True)
    lens[1] = 0
    got = O.decode(k, v, 0, q, bt, lens, offs, 0.25)
    assert np.all(got[1] == 0)
    assert np.all(np.isfinite(got))


def test_decode_invariant_under_physical_block_relabelling():
    """[P3 sec. 2.1] logical order is what matters; where blocks sit
    physically does not.  Moving every block and relabelling the tables
    leaves the output bit-identical."""
    rng = np.random.default_rng(9)
    k, v, q, bt, lens, offs = make_decode_case(rng, 4, 2, 4, 8, 4, True)
    nb = k.shape[0]
    perm = rng.permutation(nb)           # new position of old block b is perm[b]
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[perm] = k
    v2[perm] = v
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    a = O.decode(k, v, 0, q, bt, lens, offs, 0.35)
    b = O.decode(k2, v2, 0, q, bt2, lens, offs, 0.35)
    assert np.array_equal(a, b)


def test_decode_threads_do_not_change_results():
    rng = np.random.default_rng(10)
    k, v, q, bt, lens, offs = make_decode_case(rng, 6, 2, 2, 8, 4, True)
    a = O.decode(k, v, 0, q, bt, lens, offs, 0.35, num_threads=1)
    b = O.decode(k, v, 0, q, bt, lens, offs, 0.35, num_threads=5)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# prefill / append attention (causal, queries = each sequence's last tokens)
# ---------------------------------------------------------------------------
def make_prefill_case(rng, nseq, hkv, G, d, bs, bf16, max_len=40, nl=2):
    k, v, _, bt, lens, offs = make_decode_case(rng, nseq, hkv, G, d, bs, bf16, max_len, nl)
    nq = np.array([rng.integers(1, int(l) + 1) for l in lens], dtype=np.int32)
    q_start = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    qf = rng.standard_normal((int(q_start[-1]), hkv * G, d)).astype(np.float32)
    q = f32_to_bf16_bits(qf) if bf16 else qf
    return k, v, q, q_start, bt, lens, offs


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_prefill_matches_torch_sdpa_with_causal_mask(bf16, G):
    """[P2 sec. 2.4 prefill; sec. 2.3] each sequence's last n tokens attend
    causally over its gathered K/V: compared with torch's
    scaled_dot_product_attention in float64 with an explicit boolean mask
    (query i at position L - n + i sees keys 0 .. L - n + i)."""
    rng = np.random.default_rng(200 + G + 10 * bf16)
    hkv, d, bs, layer = 2, 16, 4, 1
    k, v, q, q_start, bt, lens, offs = make_prefill_case(rng, 5, hkv, G, d, bs, bf16)
    scale = 0.3
    got = O.prefill(k, v, layer, q, q_start, bt, lens, offs, scale, num_threads=3)
    for s in range(len(lens)):
        L, n = int(lens[s]), int(q_start[s + 1] - q_start[s])
        kc = to_f64(O.gather_flat_index(k[:, layer], bt[s], L, bs, int(offs[s])))
        vc = to_f64(O.gather_flat_index(v[:, layer], bt[s], L, bs, int(offs[s])))
        K = torch.from_numpy(kc).permute(1, 0, 2).repeat_interleave(G, dim=0)   # (Hq, L, D)
        V = torch.from_numpy(vc).permute(1, 0, 2).repeat_interleave(G, dim=0)
        Q = torch.from_numpy(to_f64(q[q_start[s]:q_start[s + 1]])).permute(1, 0, 2)  # (Hq, n, D)
        pos = torch.arange(L - n, L)[:, None]
        mask = torch.arange(L)[None, :] <= pos                                    # (n, L)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask,
                                                               scale=scale)
        np.testing.assert_allclose(got[q_start[s]:q_start[s + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=0, atol=1e-12)


def test_prefill_without_prefix_is_torch_causal():
    """n = L (the whole prompt is new): plain causal attention, torch's
    is_causal form."""
    rng = np.random.default_rng(21)
    hkv, G, d, bs = 2, 2, 16, 4
    k, v, _, bt, lens, offs = make_decode_case(rng, 3, hkv, G, d, bs, False)
    q_start = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = rng.standard_normal((int(q_start[-1]), hkv * G, d)).astype(np.float32)
    got = O.prefill(k, v, 0, q, q_start, bt, lens, offs, 0.4)
    for s in range(3):
        L = int(lens[s])
        kc = O.gather_flat_index(k[:, 0], bt[s], L, bs, int(offs[s])).astype(np.float64)
        vc = O.gather_flat_index(v[:, 0], bt[s], L, bs, int(offs[s])).astype(np.float64)
        K = torch.from_numpy(kc).permute(1, 0, 2).repeat_interleave(G, dim=0)
        V = torch.from_numpy(vc).permute(1, 0, 2).repeat_interleave(G, dim=0)
        Q = torch.from_numpy(q[q_start[s]:q_start[s + 1]].astype(np.float64)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=0.4)
        np.testing.assert_allclose(got[q_start[s]:q_start[s + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=0, atol=1e-12)
        # the prompt's first token sees only itself: out = V[0] exactly
        assert np.array_equal(got[q_start[s]], np.repeat(vc[0], G, axis=0))


def test_prefill_of_one_query_is_decode():
    """n = 1: the last token sees every cached token -- the decode result,
    bit for bit."""
    rng = np.random.default_rng(22)
    k, v, q, bt, lens, offs = make_decode_case(rng, 6, 2, 4, 8, 4, True)
    q_start = np.arange(7, dtype=np.int32)
    a = O.prefill(k, v, 1, q, q_start, bt, lens, offs, 0.35)
    b = O.decode(k, v, 1, q, bt, lens, offs, 0.35)
    assert np.array_equal(a, b)


def test_prefill_queries_beyond_the_sequence_are_zero():
    """More queries than cached tokens: the leading queries would sit at a
    negative position, see nothing and give zeros; the rest are unchanged."""
    rng = np.random.default_rng(23)
    k, v, _, bt, lens, offs = make_decode_case(rng, 2, 2, 2, 8, 4, False)
    L0, L1 = int(lens[0]), int(lens[1])
    q_start = np.array([0, L0 + 3, L0 + 3 + L1], np.int32)   # 3 extra queries for seq 0
    q = rng.standard_normal((L0 + 3 + L1, 4, 8)).astype(np.float32)
    got = O.prefill(k, v, 0, q, q_start, bt, lens, offs, 0.5)
    assert np.all(got[:3] == 0)
    ref = O.prefill(k, v, 0, q[3:], np.array([0, L0, L0 + L1], np.int32), bt, lens, offs, 0.5)
    assert np.array_equal(got[3:], ref)


# ---------------------------------------------------------------------------
# whole-block moves: the copy of copy-on-write, the swap of preemption
# ---------------------------------------------------------------------------
def gather_all_layers(pool, table, L, bs, off):
    return np.stack([O.gather_flat_index(pool[:, l], table, L, bs, off)
                     for l in range(pool.shape[1])])


@pytest.mark.parametrize("bs", [1, 4, 16])
def test_copy_blocks_gives_writers_the_same_tokens(bs):
    """ch. 12, 3.1 (sharing by copy-on-write): after copying each block of
    a table to a fresh block, the table remapped to the copies gathers the
    same K/V at every layer as the original, bit for bit; blocks that were
    neither source nor destination keep their bytes; a pair naming a block
    outside the pool is skipped."""
    rng = np.random.default_rng(300 + bs)
    k, _, _, bt, lens, offs = make_decode_case(rng, 3, 2, 1, 8, bs, True, max_len=30, nl=3)
    nb = k.shape[0]
    extra = rng.standard_normal((nb,) + k.shape[1:]).astype(np.float32)
    pool = np.concatenate([k, f32_to_bf16_bits(extra)])      # fresh blocks nb .. 2nb-1
    used = sorted({int(b) for b in bt[bt >= 0]})
    dst = [nb + i for i in range(len(used))]
    before = pool.copy()
    O.copy_blocks(pool, used + [2 * nb + 5], dst + [0])
    remap = {s: d for s, d in zip(used, dst)}
    for s in range(3):
        L, off = int(lens[s]), int(offs[s])
        t2 = np.array([remap.get(int(b), -1) for b in bt[s]], np.int32)
        assert np.array_equal(gather_all_layers(pool, t2, L, bs, off),
                              gather_all_layers(before, bt[s], L, bs, off))
    untouched = [b for b in range(2 * nb) if b not in dst]
    assert np.array_equal(pool[untouched], before[untouched])


def test_swap_out_holds_each_blocks_tokens_and_swap_in_restores_them():
    """P2 2.4 (preemption swaps KV GPU -> CPU and back): swap_out's i-th
    entry at layer l is what a one-block table gathers at layer l (all bs
    slots); swapping those blocks back in at other ids gives the same gather
    through the remapped table as the original, bit for bit."""
    rng = np.random.default_rng(31)
    bs = 4
    k, _, _, bt, lens, offs = make_decode_case(rng, 2, 2, 1, 8, bs, False, max_len=20, nl=2)
    nb = k.shape[0]
    ids = [int(b) for b in bt[0] if b >= 0]
    host = O.swap_out(k, ids)
    assert host.shape == (len(ids),) + k.shape[1:]
    for i, b in enumerate(ids):
        one = np.array([b], np.int32)
        assert np.array_equal(host[i], gather_all_layers(k, one, bs, bs, 0))
    pool = np.concatenate([k, np.zeros_like(k)])
    new_ids = [nb + i for i in range(len(ids))]
    O.swap_in(pool, new_ids, host)
    t2 = np.array([nb + ids.index(int(b)) if b >= 0 else -1 for b in bt[0]], np.int32)
    L, off = int(lens[0]), int(offs[0])
    assert np.array_equal(gather_all_layers(pool, t2, L, bs, off),
                          gather_all_layers(k, bt[0], L, bs, off))
    with pytest.raises(ValueError):
        O.swap_out(k, [nb])
