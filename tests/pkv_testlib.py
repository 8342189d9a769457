"""Helpers shared by the GPU parity tests: host copies for the oracle,
compact pools, and the comparison bars.

Compact pools: the full 16384-block, 32-layer pools are 16 GiB per tensor,
so the oracle is handed only the blocks the tables reference, at the layer
under test: pool[ids, layer] with the tables renumbered to positions in
`ids`.  Renumbering blocks does not change what a gather or a decode reads
(logical order is all that matters), so the oracle's answer on the compact
copy is its answer on the full pool.
"""
import os

import numpy as np
import torch

import oracle as O

# Decode tolerance (max abs error vs the float64 oracle): bf16 inputs with
# fp32 accumulation, and fp32 inputs.
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-5}


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def host(t: torch.Tensor) -> np.ndarray:
    """Bit-exact host copy: bf16 becomes uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def compact(k_pool, v_pool, layer, block_tables):
    """(k_c, v_c, tables_c, ids): host pools (len(ids), 1, bs, H, D) holding
    the referenced blocks at `layer`, tables renumbered into them."""
    bt = block_tables.cpu()
    ids = torch.unique(bt[bt >= 0]).to(torch.int64)
    dev_ids = ids.to(k_pool.device)
    k_c = host(k_pool[:, layer].index_select(0, dev_ids).unsqueeze(1))
    v_c = None if v_pool is None else host(v_pool[:, layer].index_select(0, dev_ids).unsqueeze(1))
    pos = torch.searchsorted(ids, bt.clamp(min=0).to(torch.int64)).to(torch.int32)
    tables_c = torch.where(bt >= 0, pos, torch.full_like(pos, -1)).numpy()
    return k_c, v_c, tables_c, ids


def oracle_decode_for(w, q=None, seqs=None):
    """Oracle decode of workload w (optionally only sequences `seqs`)."""
    q = w.q if q is None else q
    bt, sl, off = w.block_tables, w.seq_lens, w.offsets
    if seqs is not None:
        idx = torch.as_tensor(seqs, dtype=torch.int64, device=bt.device)
        bt, sl, off = bt[idx], sl[idx], off[idx]
        q = q[idx.to(q.device)]
    k_c, v_c, bt_c, _ = compact(w.k_pool, w.v_pool, w.layer, bt)
    return O.decode(k_c, v_c, 0, host(q), bt_c, host(sl), host(off), w.scale,
                    num_threads=oracle_threads())


def max_abs_err(got: torch.Tensor, ref: np.ndarray) -> float:
    g = as_f64(got)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    if not np.all(np.isfinite(g)):
        return float("inf")
    return float(np.max(np.abs(g - ref))) if g.size else 0.0


def row_starts(seq_lens: torch.Tensor) -> torch.Tensor:
    """Exclusive prefix sum of seq_lens as int64 (output row of each seq)."""
    sl = seq_lens.to(torch.int64)
    return torch.cumsum(sl, 0) - sl
