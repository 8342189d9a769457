"""Pins of the quantised-KV oracle (oracle/quant.py).

The pages name quantised KV (int8 / int4) as the next compression step of a
paged cache (mini-runtime ch. 12, sec. 6 evolution diagram) and give no
method, so the oracle takes the plain symmetric reading: one float32 scale
amax / 127 per (token, kv head) row, codes = round-half-even(x / scale).
These tests pin that reading by mathematics and by the already pinned
gather and decode:

  * every stored value is within half a quantisation step of the input, the
    row's largest magnitude maps to +-127, and integer rows of amax 127 come
    back exactly (scale 1); rounding ties go to even;
  * codes are odd-symmetric and invariant under power-of-two scaling;
  * gather over the quantised pool equals a per-token loop over the stated
    layouts;
  * decode over the quantised pool equals the C oracle's decode of a float32
    pool holding the same values, when those values are exact in float32
    (power-of-two scales), and stays within float32 rounding otherwise.

Planted mistakes (floor rounding, amax / 128, one scale per token over all
heads, ties away from zero, scales read transposed) each fail a pin.
"""
import numpy as np
import pytest

import oracle as O
from oracle import quant as Q


def rows(rng, n, h, d, lo=-3, hi=3):
    """Rows with magnitudes spread over 10^lo .. 10^hi per row."""
    mag = 10.0 ** rng.uniform(lo, hi, size=(n, h, 1))
    return (rng.standard_normal((n, h, d)) * mag).astype(np.float32)


def check_reading(quantize, x):
    """The facts the reading fixes, for one quantiser; returns failures."""
    bad = []
    c, s = quantize(x)
    amax = np.max(np.abs(x), axis=-1)
    if not np.array_equal(s, (amax / np.float32(127)).astype(np.float32)):
        bad.append("scale")
    err = np.abs(Q.dequantize_f64(c, s) - x.astype(np.float64))
    if np.any(err > s.astype(np.float64)[..., None] * (0.5 + 2.0 ** -20)):
        bad.append("half-step bound")
    if np.any(np.abs(c.astype(np.int32)) > 127):
        bad.append("code range")
    top = np.take_along_axis(np.abs(c.astype(np.int32)), np.argmax(np.abs(x), -1)[..., None], -1)
    if np.any(top[..., 0][amax > 0] != 127):
        bad.append("amax code")
    ints = np.array([[127, 2.5, -3.5, 0.5, -0.5, 1.5, -127, 40]], np.float32)
    ci, si = quantize(ints)
    if not (si[0] == 1.0 and list(ci[0]) == [127, 2, -4, 0, 0, 2, -127, 40]):
        bad.append("ties to even / exact integers")
    return bad


def test_quantize_meets_the_reading():
    rng = np.random.default_rng(1)
    x = rows(rng, 300, 4, 128)
    assert check_reading(Q.quantize_rows, x) == []
    # bf16 inputs (bit patterns) quantise their float32 values
    b = Q.bf16_bits(x)
    c1, s1 = Q.quantize_rows(b)
    c2, s2 = Q.quantize_rows(Q.as_f32(b))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_quantize_zero_rows_symmetry_and_power_of_two_scaling():
    rng = np.random.default_rng(2)
    x = rows(rng, 50, 2, 64)
    x[3, 1] = 0.0
    c, s = Q.quantize_rows(x)
    assert s[3, 1] == 0 and not c[3, 1].any()
    cn, sn = Q.quantize_rows(-x)
    assert np.array_equal(cn, -c) and np.array_equal(sn, s)
    for k in (-7, 5):
        ck, sk = Q.quantize_rows(x * np.float32(2.0 ** k))
        assert np.array_equal(ck, c) and np.array_equal(sk, s * np.float32(2.0 ** k))


def _floor(x):
    c, s = Q.quantize_rows(x)
    div = np.where(s > 0, s, 1)[..., None]
    return np.clip(np.floor(x / div), -127, 127).astype(np.int8), s


def _over_128(x):
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(128)).astype(np.float32)
    div = np.where(s > 0, s, 1)[..., None]
    return np.clip(np.rint(x / div), -127, 127).astype(np.int8), s


def _one_scale_per_token(x):
    amax = np.max(np.abs(x.reshape(x.shape[0], -1)), axis=-1)
    s = (amax / np.float32(127)).astype(np.float32).reshape((-1,) + (1,) * (x.ndim - 2))
    s = np.broadcast_to(s, x.shape[:-1])
    div = np.where(s > 0, s, 1)[..., None]
    return np.clip(np.rint(x / div), -127, 127).astype(np.int8), np.ascontiguousarray(s)


def _ties_away(x):
    c, s = Q.quantize_rows(x)
    div = np.where(s > 0, s, 1)[..., None].astype(np.float32)
    t = (x / div).astype(np.float32)
    return np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -127, 127).astype(np.int8), s


@pytest.mark.parametrize("mutant", [_floor, _over_128, _one_scale_per_token, _ties_away],
                         ids=lambda f: f.__name__)
def test_planted_quantiser_mistake_fails(mutant):
    rng = np.random.default_rng(3)
    x = rows(rng, 40, 4, 64)
    assert check_reading(mutant, x)


def make_pool(rng, nb, nl, bs, h, d, pow2):
    codes = rng.integers(-127, 128, size=(nb, nl, bs, h, d)).astype(np.int8)
    if pow2:
        scales = (2.0 ** rng.integers(-12, 4, size=(nb, nl, h, bs))).astype(np.float32)
    else:
        scales = (10.0 ** rng.uniform(-3, 0, size=(nb, nl, h, bs))).astype(np.float32)
    return codes, scales


def tables(rng, nseq, bs, nb, max_len):
    lens = rng.integers(0, max_len + 1, size=nseq).astype(np.int32)
    offs = rng.integers(0, bs, size=nseq).astype(np.int32)
    need = [O.blocks_needed(int(l) + int(o), bs) for l, o in zip(lens, offs)]
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((nseq, max(max(need), 1)), -1, np.int32)
    at = 0
    for i, c in enumerate(need):
        bt[i, :c] = perm[at:at + c]
        at += c
    return bt, lens, offs


def test_gather_q8_is_the_per_token_definition():
    """Token t of a sequence sits at flat position off + t of its table
    (P3 sec. 2.2); its stored row at kv head h is codes[b, l, r, h] *
    scales[b, l, h, r] (float32), rounded to bf16."""
    rng = np.random.default_rng(4)
    bs, h, d, nl = 4, 3, 64, 2
    bt, lens, offs = tables(rng, 4, bs, 64, 30)
    codes, scales = make_pool(rng, 64, nl, bs, h, d, pow2=False)
    got = Q.gather_q8(codes, scales, 1, bt, lens, offs)
    want = []
    for s in range(4):
        for t in range(int(lens[s])):
            p = int(offs[s]) + t
            b, r = int(bt[s, p // bs]), p % bs
            row = codes[b, 1, r].astype(np.float32) * scales[b, 1, :, r][:, None]
            want.append(Q.bf16_bits(row.astype(np.float32)))
    assert np.array_equal(got, np.array(want).reshape(got.shape))
    # scales read as (.., bs, H) instead of (.., H, bs) change the answer
    wrong = np.ascontiguousarray(scales.reshape(64, nl, bs, h).transpose(0, 1, 3, 2))
    assert not np.array_equal(Q.gather_q8(codes, wrong, 1, bt, lens, offs), got)


def test_scatter_q8_then_gather_q8():
    """Rows scattered with quantisation come back as bf16(code * scale) of
    their own quantisation; slot -1 rows are dropped; every other byte of
    the pool is unchanged."""
    rng = np.random.default_rng(5)
    nb, nl, bs, h, d = 12, 2, 4, 2, 64
    codes, scales = make_pool(rng, nb, nl, bs, h, d, pow2=False)
    c0, s0 = codes.copy(), scales.copy()
    x = rows(rng, 9, h, d)
    slots = np.array([5, 6, -1, 7, 8, 9, 10, 11, 40], np.int64)
    Q.scatter_q8(codes, scales, 1, x, slots)
    cq, sq = Q.quantize_rows(x)
    for i, sl in enumerate(slots.tolist()):
        if sl >= 0:
            assert np.array_equal(codes[sl // bs, 1, sl % bs], cq[i])
            assert np.array_equal(scales[sl // bs, 1, :, sl % bs], sq[i])
    touched = np.zeros((nb, nl, bs), bool)
    for sl in slots[slots >= 0].tolist():
        touched[sl // bs, 1, sl % bs] = True
    assert np.array_equal(codes[~touched], c0[~touched])
    assert np.array_equal(scales.transpose(0, 1, 3, 2)[~touched], s0.transpose(0, 1, 3, 2)[~touched])
    # one sequence over slots 5..11 (blocks 1, 2; offset 1): its gather
    bt = np.array([[1, 2]], np.int32)
    got = Q.gather_q8(codes, scales, 1, bt, np.array([7], np.int32), np.array([1], np.int32))
    # tokens 0..6 sit at slots 5..11, which hold rows 0, 1, 3, 4, 5, 6, 7
    # (row 2 was dropped)
    keep = [0, 1, 3, 4, 5, 6, 7]
    assert np.array_equal(got, Q.bf16_bits(Q.dequantize_f32(cq[keep], sq[keep])))
    with pytest.raises(ValueError):
        Q.scatter_q8(codes, scales, 0, x[:1], np.array([nb * bs], np.int64))


@pytest.mark.parametrize("G", [1, 4])
def test_decode_q8_is_decode_of_the_stored_values(G):
    """With power-of-two scales the stored values are exact in float32, so
    decode over the quantised pool must equal the C oracle's decode of a
    float32 pool holding them (both float64 inside); with other scales the
    two differ only by the float32 rounding of the stored values."""
    rng = np.random.default_rng(6 + G)
    nb, nl, bs, hkv, d = 48, 2, 4, 2, 64
    bt, lens, offs = tables(rng, 5, bs, nb, 30)
    q = rng.standard_normal((5, hkv * G, d)).astype(np.float32)
    for pow2 in (True, False):
        kc, ks = make_pool(rng, nb, nl, bs, hkv, d, pow2)
        vc, vs = make_pool(rng, nb, nl, bs, hkv, d, pow2)
        kf = Q.dequantize_f32(kc, ks.transpose(0, 1, 3, 2))
        vf = Q.dequantize_f32(vc, vs.transpose(0, 1, 3, 2))
        got = Q.decode_q8(kc, ks, vc, vs, 1, q, bt, lens, offs, 0.125)
        ref = O.decode(kf, vf, 1, q, bt, lens, offs, 0.125)
        tol = 1e-12 if pow2 else 1e-5
        assert np.max(np.abs(got - ref)) <= tol * max(1.0, np.max(np.abs(ref)))
    assert not got[lens == 0].any()
