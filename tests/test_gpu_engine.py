"""The native block manager driving the kernels through a decode loop.

Requests arrive (allocate with a random first-block offset, then write the
prompt rows with kv_append through the manager's table), every step gives
each live request one new token (append_slots, then kv_scatter of its rows
to those slots), some requests finish (free) and later ones reuse their
blocks.  At the end the pool holds, for every live request, exactly the
rows it was given, in order (kv_gather over the manager's tables, bit for
bit), and paged_attn_decode over those tables matches the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from paged_attention_decode_scatter_amd import native as N
from tests.pkv_testlib import TOL, host, max_abs_err, row_starts

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.load_library()
    return torch.device("cuda:0")


def test_block_manager_drives_append_scatter_gather_decode(dev):
    rng = np.random.default_rng(9)
    gen = torch.Generator(device=dev).manual_seed(9)
    nb, nl, bs, hkv, d, hq, layer = 384, 2, 16, 2, 128, 8, 1
    k_pool = torch.zeros((nb, nl, bs, hkv, d), dtype=torch.bfloat16, device=dev)
    v_pool = torch.zeros_like(k_pool)
    m = N.BlockManager(nb, bs)
    rows = {}        # seq -> list of (k, v) rows [hkv, d], in token order
    next_id = 0

    def rand_rows(n):
        shape = (n, hkv, d)
        return (torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16),
                torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16))

    def arrive():
        nonlocal next_id
        ln = int(rng.integers(1, 200))
        off = int(rng.integers(0, bs))
        if not m.allocate(next_id, ln, off):
            return
        tab, _, offs = m.tables([next_id])
        k, v = rand_rows(ln)
        N.kv_append(k_pool, v_pool, layer, k, v, torch.from_numpy(tab).to(dev),
                    torch.from_numpy(offs).to(dev),
                    torch.zeros(ln, dtype=torch.int32, device=dev),
                    torch.arange(ln, dtype=torch.int32, device=dev))
        rows[next_id] = [(k[i], v[i]) for i in range(ln)]
        next_id += 1

    for _ in range(6):
        arrive()
    refused = 0
    for step in range(40):
        if rng.random() < 0.3:
            arrive()
        live = sorted(rows)
        n, slots = m.append_slots(live)
        refused += len(live) - n
        if n:
            k, v = rand_rows(n)
            N.kv_scatter(k_pool, v_pool, layer, k, v, torch.from_numpy(slots[:n]).to(dev))
            for i, q in enumerate(live[:n]):
                rows[q].append((k[i], v[i]))
        if rng.random() < 0.15 and len(live) > 2:
            q = int(rng.choice(live))
            m.free(q)
            del rows[q]
    torch.cuda.synchronize()
    live = sorted(rows)
    assert len(live) >= 3
    st = m.stats()
    assert st["live_tokens"] == sum(len(r) for r in rows.values())

    tab, lens, offs = m.tables(live)
    bt = torch.from_numpy(tab).to(dev)
    sl = torch.from_numpy(lens).to(dev)
    of = torch.from_numpy(offs).to(dev)
    total = int(lens.sum())
    k_out = torch.empty((total, hkv, d), dtype=torch.bfloat16, device=dev)
    v_out = torch.empty_like(k_out)
    N.kv_gather(k_pool, v_pool, layer, bt, sl, of, row_starts(sl), int(lens.max()), k_out, v_out)
    torch.cuda.synchronize()
    k_exp = torch.stack([r[0] for q in live for r in rows[q]])
    v_exp = torch.stack([r[1] for q in live for r in rows[q]])
    assert torch.equal(k_out.view(torch.int16), k_exp.view(torch.int16))
    assert torch.equal(v_out.view(torch.int16), v_exp.view(torch.int16))

    q = torch.randn((len(live), hq, d), generator=gen, device=dev).to(torch.bfloat16)
    scale = 1.0 / np.sqrt(d)
    for split in (0, 64, N.SPLIT_PLANNED):
        out = N.paged_attn_decode(k_pool, v_pool, layer, q, bt, sl, of, int(lens.max()), scale,
                                  split_tokens=split)
        ref = O.decode(host(k_pool), host(v_pool), layer, host(q), tab, lens, offs, scale)
        assert max_abs_err(out, ref) <= TOL[torch.bfloat16], split
