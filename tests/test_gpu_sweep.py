"""A seeded random sweep of small cases through the C ABI against the oracle,
reaching combinations the fixed grids of the other tests do not: pool dtype
(fp32, bf16, int8, int4) x head_dim (64, 128) x kv heads (1, 2, 3, 4, 6, 8)
x group (1, 2, 4, 8) x block size (1 .. 64) x split (automatic, planned,
16 .. 256), with random first-block offsets and some empty sequences.  For
every case: the gather is bit-exact and decode is within the dtype's
tolerance of the oracle's float64 decode.
"""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import quant as Q
from paged_attention_decode_scatter_amd import native as N
from paged_attention_decode_scatter_amd import workloads as W
from tests.pkv_testlib import TOL, host, max_abs_err, oracle_decode_for, row_starts

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "bf16", "i8", "i4"]
QTOL = 2e-2


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.load_library()
    return torch.device("cuda:0")


def case(seed):
    r = np.random.default_rng(7000 + seed)
    return dict(dtype=DTYPES[r.integers(4)], d=int(r.choice([64, 128])),
                hkv=int(r.choice([1, 2, 3, 4, 6, 8])), g=int(r.choice([1, 2, 4, 8])),
                bs=int(r.choice([1, 2, 4, 8, 16, 32, 64])), n=int(r.integers(1, 11)),
                max_len=int(r.integers(1, 600)),
                split=int(r.choice([0, N.SPLIT_PLANNED, 16, 48, 64, 128, 256])), seed=seed)


def build(dev, c):
    counts_max = (c["max_len"] + c["bs"] - 1) // c["bs"] + 1
    nb = c["n"] * counts_max + 16
    fdt = torch.float32 if c["dtype"] == "f32" else torch.bfloat16
    quant = c["dtype"] in ("i8", "i4")
    w = W.decode_batch(device=dev, seed=8000 + c["seed"], num_seqs=c["n"], min_len=0,
                       max_len=c["max_len"], num_blocks=nb, num_layers=2, num_kv_heads=c["hkv"],
                       head_dim=c["d"], num_q_heads=c["hkv"] * c["g"], dtype=fdt, layer=1,
                       offsets="random", block_size=c["bs"], with_pools=not quant)
    if quant:
        make = W.int8_pool_tensors if c["dtype"] == "i8" else W.int4_pool_tensors
        shape = (nb, 2, c["bs"], c["hkv"], c["d"])
        w.k_pool = N.QuantizedPool(*make(*shape, dev, 8100 + c["seed"]))
        w.v_pool = N.QuantizedPool(*make(*shape, dev, 8200 + c["seed"]))
    return w


@pytest.mark.parametrize("seed", range(48))
def test_random_case(dev, seed):
    c = case(seed)
    print(c, flush=True)
    w = build(dev, c)
    quant = c["dtype"] in ("i8", "i4")
    args = (w.layer, host(w.block_tables), host(w.seq_lens), host(w.offsets))
    # gather, bit-exact
    rows = int(w.seq_lens.sum())
    odt = torch.float32 if c["dtype"] == "f32" else torch.bfloat16
    ko = torch.full((max(rows, 1), c["hkv"], c["d"]), float("nan"), dtype=odt, device=dev)[:rows]
    vo = torch.full_like(ko, float("nan"))
    if rows:
        N.kv_gather(w.k_pool, w.v_pool, w.layer, w.block_tables, w.seq_lens, w.offsets,
                    row_starts(w.seq_lens), w.max_seq_len, ko, vo)
        torch.cuda.synchronize()
        if quant:
            gq = Q.gather_q8 if c["dtype"] == "i8" else Q.gather_q4
            assert np.array_equal(host(ko), gq(host(w.k_pool.codes), host(w.k_pool.scales), *args))
            assert np.array_equal(host(vo), gq(host(w.v_pool.codes), host(w.v_pool.scales), *args))
        else:
            assert np.array_equal(host(ko).view(np.uint8), O.gather(host(w.k_pool), *args).view(np.uint8))
            assert np.array_equal(host(vo).view(np.uint8), O.gather(host(w.v_pool), *args).view(np.uint8))
    # decode (a planned split the batch cannot take is refused: then the automatic one)
    out = torch.full_like(w.q, float("nan"))
    try:
        got = N.paged_attn_decode(w.k_pool, w.v_pool, w.layer, w.q, w.block_tables, w.seq_lens,
                                  w.offsets, w.max_seq_len, w.scale, split_tokens=c["split"],
                                  out=out)
    except N.PagedKVError as e:
        assert c["split"] == N.SPLIT_PLANNED and e.status == -8, e   # PKV_ERR_UNSUPPORTED
        got = N.paged_attn_decode(w.k_pool, w.v_pool, w.layer, w.q, w.block_tables, w.seq_lens,
                                  w.offsets, w.max_seq_len, w.scale, split_tokens=0, out=out)
    torch.cuda.synchronize()
    if quant:
        dq = Q.decode_q8 if c["dtype"] == "i8" else Q.decode_q4
        want = dq(host(w.k_pool.codes), host(w.k_pool.scales), host(w.v_pool.codes),
                  host(w.v_pool.scales), w.layer, host(w.q), *args[1:], w.scale)
        assert max_abs_err(got, want) <= QTOL
    else:
        assert max_abs_err(got, oracle_decode_for(w)) <= TOL[odt]
