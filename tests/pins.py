"""Pins for the float64 oracle: facts fixed by the mathematics, not by the oracle.

Each pin takes an implementation namespace `impl` (the oracle package, or a
mutant of it built in tests/test_oracle_mutants.py) and raises AssertionError
when `impl` disagrees with the fact. The pins are chosen so that a plausible
slip anywhere in the oracle (a dropped scale, a wrong mask bound, a wrong
head or user index, the wrong operand or reduction axis) fails at least one.
"""
from __future__ import annotations

import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(shape, seed):
    return _rng(seed).standard_normal(shape)


# --- exact worked example ---------------------------------------------------

def pin_golden_rational(impl):
    """Hand-derived rational outputs (tests/golden/rational_case.json)."""
    with open(os.path.join(GOLDEN, "rational_case.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], float)[None, None]
    k = np.array(g["k"], float)[None, None]
    v = np.array(g["v"], float)[None, None]
    for case in g["cases"]:
        kv = None if case["kv_len"] is None else np.array([case["kv_len"]])
        o = impl.attention(q, k, v, causal=case["causal"], kv_len=kv, scale=math.log(2))
        want = np.array([[float(Fraction(x)) for x in row] for row in case["o"]])
        np.testing.assert_allclose(o[0, 0], want, rtol=0, atol=1e-14, err_msg=str(case))


# --- closed forms -------------------------------------------------------------

def pin_two_key_sigmoid(impl):
    """Two keys: o = sigma(D) v0 + sigma(-D) v1 with D = scale (q.k0 - q.k1)."""
    d = 8
    q, k, v = _rand((2, 3, 5, d), 1), _rand((2, 3, 2, d), 2), _rand((2, 3, 2, d), 3)
    sc = 0.37
    o = impl.attention(q, k, v, scale=sc)
    for b in range(2):
        for h in range(3):
            for i in range(5):
                D = sc * (float(np.dot(q[b, h, i], k[b, h, 0])) - float(np.dot(q[b, h, i], k[b, h, 1])))
                w0 = 0.5 * (1.0 + math.tanh(D / 2))
                want = w0 * v[b, h, 0] + (1.0 - w0) * v[b, h, 1]
                np.testing.assert_allclose(o[b, h, i], want, rtol=0, atol=1e-13)


def pin_default_scale(impl):
    """scale None and 0 both mean 1/sqrt(d) (checked on two keys, closed form)."""
    d = 16
    q, k, v = _rand((1, 1, 3, d), 4), _rand((1, 1, 2, d), 5), _rand((1, 1, 2, d), 6)
    for s in (None, 0.0):
        o = impl.attention(q, k, v, scale=s)
        for i in range(3):
            D = (float(np.dot(q[0, 0, i], k[0, 0, 0])) - float(np.dot(q[0, 0, i], k[0, 0, 1]))) / math.sqrt(d)
            w0 = 0.5 * (1.0 + math.tanh(D / 2))
            np.testing.assert_allclose(o[0, 0, i], w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, 1],
                                       rtol=0, atol=1e-13)


def pin_constant_v(impl):
    """Every v_j equal to c gives o = c for every row with a valid key."""
    B, H, L, d = 2, 2, 9, 4
    q, k = _rand((B, H, L, d), 7), _rand((B, H, L, d), 8)
    c = _rand((d,), 9)
    v = np.broadcast_to(c, (B, H, L, d)).copy()
    for causal in (False, True):
        for kv in (None, np.array([9, 3])):
            o = impl.attention(q, k, v, causal=causal, kv_len=kv)
            np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-14)


def pin_single_key(impl):
    """Lk = 1: o = v_0 whatever q, k and the scale are."""
    q, k, v = _rand((2, 4, 6, 8), 10), _rand((2, 2, 1, 8), 11), _rand((2, 2, 1, 8), 12)
    o = impl.attention(q, k, v, scale=3.0)
    want = np.repeat(v, 2, axis=1)  # heads 0,1 -> kv 0; heads 2,3 -> kv 1
    np.testing.assert_allclose(o, np.broadcast_to(want, o.shape), rtol=0, atol=1e-14)


def pin_zero_query_mean(impl):
    """q = 0: all valid scores are equal, so o is the plain mean of the valid v_j.

    With causal (top-left) row i sees keys 0..i; with kv_len n sees keys 0..n-1.
    """
    B, H, Lq, Lk, d = 2, 1, 7, 6, 3
    q = np.zeros((B, H, Lq, d))
    k, v = _rand((B, H, Lk, d), 13), _rand((B, H, Lk, d), 14)
    kv = np.array([4, 6])
    for causal in (False, True):
        o = impl.attention(q, k, v, causal=causal, kv_len=kv)
        for b in range(B):
            for i in range(Lq):
                n = kv[b] if not causal else min(kv[b], i + 1)
                np.testing.assert_allclose(o[b, 0, i], v[b, 0, :n].mean(axis=0), rtol=0, atol=1e-14)


def pin_fully_masked_zero(impl):
    """kv_len = 0 leaves no valid key: the output row is exactly 0."""
    q, k, v = _rand((2, 2, 5, 4), 15), _rand((2, 2, 5, 4), 16), _rand((2, 2, 5, 4), 17)
    o = impl.attention(q, k, v, kv_len=np.array([0, 5]))
    assert np.all(o[0] == 0.0)
    assert np.all(np.abs(o[1]) > 0)


def pin_causal_first_row(impl):
    """Causal row 0 sees key 0 only: o[.,.,0] = v_0 exactly."""
    q, k, v = _rand((2, 4, 5, 8), 18), _rand((2, 2, 7, 8), 19), _rand((2, 2, 7, 8), 20)
    o = impl.attention(q, k, v, causal=True)
    np.testing.assert_allclose(o[:, :, 0], np.repeat(v[:, :, 0], 2, axis=1), rtol=0, atol=1e-15)


def pin_hard_max_limit(impl):
    """Large scale with distinct logits: softmax -> one-hot at argmax_j q.k_j."""
    q, k, v = _rand((1, 2, 6, 8), 21), _rand((1, 2, 9, 8), 22), _rand((1, 2, 9, 8), 23)
    o = impl.attention(q, k, v, scale=1e4)
    for h in range(2):
        for i in range(6):
            j = int(np.argmax(k[0, h] @ q[0, h, i]))
            np.testing.assert_allclose(o[0, h, i], v[0, h, j], rtol=0, atol=1e-12)


# --- invariants -----------------------------------------------------------------

def pin_probabilities_rows(impl):
    """P rows sum to 1 over valid keys; masked entries are exactly 0."""
    q, k, v = _rand((2, 2, 8, 4), 24), _rand((2, 2, 8, 4), 25), _rand((2, 2, 8, 4), 26)
    kv = np.array([5, 8])
    for causal in (False, True):
        for b in range(2):
            p = impl.probabilities(q, k, v, causal=causal, kv_len=kv, b=b, h=1)
            np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
            i, j = np.meshgrid(np.arange(8), np.arange(8), indexing="ij")
            masked = (j >= kv[b]) | ((j > i) if causal else False)
            assert np.all(p[masked] == 0.0) and np.all(p[~masked] > 0.0)


def pin_key_permutation(impl):
    """No mask: permuting the keys and values together leaves o unchanged."""
    q, k, v = _rand((2, 2, 5, 8), 27), _rand((2, 2, 11, 8), 28), _rand((2, 2, 11, 8), 29)
    perm = _rng(30).permutation(11)
    o1 = impl.attention(q, k, v)
    o2 = impl.attention(q, k[:, :, perm], v[:, :, perm])
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)


def pin_key_shift(impl):
    """k_j += w for all j adds the same constant to a row's scores: o unchanged."""
    q, k, v = _rand((1, 2, 6, 8), 31), _rand((1, 2, 6, 8), 32), _rand((1, 2, 6, 8), 33)
    w = _rand((8,), 34)
    for causal in (False, True):
        o1 = impl.attention(q, k, v, causal=causal, kv_len=np.array([4]))
        o2 = impl.attention(q, k + w, v, causal=causal, kv_len=np.array([4]))
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)


def pin_scale_homogeneity(impl):
    """attention(a*q, scale=s) equals attention(q, scale=a*s)."""
    q, k, v = _rand((1, 2, 5, 8), 35), _rand((1, 2, 7, 8), 36), _rand((1, 2, 7, 8), 37)
    o1 = impl.attention(2.5 * q, k, v, scale=0.2)
    o2 = impl.attention(q, k, v, scale=0.5)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)


def pin_gqa_is_head_repeat(impl):
    """GQA equals multi-head attention with each K/V head repeated H/Hkv times
    in contiguous groups (query head h uses K/V head h // (H/Hkv))."""
    q, k, v = _rand((2, 6, 5, 4), 38), _rand((2, 2, 7, 4), 39), _rand((2, 2, 7, 4), 40)
    for causal in (False, True):
        o1 = impl.attention(q, k, v, causal=causal)
        o2 = impl.attention(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), causal=causal)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    # the grouped heads must really differ from an interleaved (h % Hkv) map
    o_wrong = impl.attention(q, np.tile(k, (1, 3, 1, 1)), np.tile(v, (1, 3, 1, 1)))
    assert np.abs(impl.attention(q, k, v) - o_wrong).max() > 1e-3


def pin_kv_len_is_truncation(impl):
    """kv_len = n equals dense attention over the first n keys; kv_len = Lk equals no mask."""
    q, k, v = _rand((3, 2, 6, 4), 41), _rand((3, 2, 9, 4), 42), _rand((3, 2, 9, 4), 43)
    kv = np.array([1, 5, 9])
    for causal in (False, True):
        o = impl.attention(q, k, v, causal=causal, kv_len=kv)
        for b, n in enumerate(kv):
            ref = impl.attention(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], causal=causal)
            np.testing.assert_allclose(o[b:b + 1], ref, rtol=0, atol=1e-14)
    o_full = impl.attention(q, k, v, kv_len=np.array([9, 9, 9]))
    np.testing.assert_allclose(o_full, impl.attention(q, k, v), rtol=0, atol=0)
    o_over = impl.attention(q, k, v, kv_len=np.array([50, -3, 9]))  # clamped to [0, Lk]
    np.testing.assert_allclose(o_over[0], impl.attention(q, k, v)[0], rtol=0, atol=0)
    assert np.all(o_over[1] == 0.0)


def pin_bcast_is_replication(impl):
    """Broadcast equals explicit replication k[cand2user], v[cand2user] (bit-equal);
    an out-of-range user index yields NaN rows."""
    B_c, B_u = 7, 3
    q = _rand((B_c, 4, 5, 8), 44)
    k, v = _rand((B_u, 2, 6, 8), 45), _rand((B_u, 2, 6, 8), 46)
    c2u = np.array([2, 0, 0, 1, 2, 1, 0])
    kv = np.array([6, 2, 4])
    for causal in (False, True):
        o1 = impl.attention_bcast(q, k, v, c2u, causal=causal, kv_len=kv)
        o2 = impl.attention(q, k[c2u], v[c2u], causal=causal, kv_len=kv[c2u])
        assert np.array_equal(o1, o2)
    bad = c2u.copy()
    bad[3] = B_u
    o3 = impl.attention_bcast(q, k, v, bad)
    assert np.all(np.isnan(o3[3])) and not np.any(np.isnan(np.delete(o3, 3, axis=0)))
    sub = impl.attention_bcast(q, k, v, c2u, cands=[4, 1], rows=[3, 0])
    full = impl.attention_bcast(q, k, v, c2u)
    np.testing.assert_array_equal(sub, full[[4, 1]][:, :, [3, 0]])


def pin_rows_subset(impl):
    """attention_rows returns exactly the requested rows of attention()."""
    q, k, v = _rand((2, 4, 9, 8), 47), _rand((2, 2, 9, 8), 48), _rand((2, 2, 9, 8), 49)
    kv = np.array([7, 3])
    for causal in (False, True):
        full = impl.attention(q, k, v, causal=causal, kv_len=kv)
        rows = np.array([8, 0, 4])
        for b in range(2):
            for h in range(4):
                part = impl.attention_rows(q, k, v, b, h, rows, causal=causal, kv_len=kv)
                np.testing.assert_array_equal(part, full[b, h, rows])


# --- brute force ------------------------------------------------------------------

def _brute_decimal(q, k, v, causal, kv_len, scale):
    """Direct 40-digit evaluation: exp of the raw scores (no max shift), explicit loops."""
    getcontext().prec = 40
    B, H, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    sc = Decimal(repr(scale))
    o = np.zeros(q.shape)
    for b in range(B):
        for h in range(H):
            g = (h * Hkv) // H
            for i in range(Lq):
                ws, num = [], [Decimal(0)] * d
                for j in range(Lk):
                    if causal and j > i:
                        continue
                    if kv_len is not None and j >= kv_len[b]:
                        continue
                    s = sum(Decimal(repr(float(q[b, h, i, t]))) * Decimal(repr(float(k[b, g, j, t])))
                            for t in range(d))
                    w = (sc * s).exp()
                    ws.append(w)
                    for t in range(d):
                        num[t] += w * Decimal(repr(float(v[b, g, j, t])))
                z = sum(ws, Decimal(0))
                if z > 0:
                    o[b, h, i] = [float(x / z) for x in num]
    return o


def pin_brute_force(impl):
    """Tiny shapes, every mask combination and GQA: 40-digit brute force."""
    q, k, v = _rand((2, 4, 5, 3), 50), _rand((2, 2, 6, 3), 51), _rand((2, 2, 6, 3), 52)
    for causal in (False, True):
        for kv in (None, np.array([6, 2])):
            for sc in (0.7, 1.0 / math.sqrt(3)):
                o = impl.attention(q, k, v, causal=causal, kv_len=kv, scale=sc)
                ref = _brute_decimal(q, k, v, causal, kv, sc)
                np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


# --- library special case -------------------------------------------------------------

def pin_torch_sdpa(impl):
    """PyTorch's float64 CPU scaled_dot_product_attention on the cases it expresses."""
    import torch
    import torch.nn.functional as F
    q, k, v = _rand((2, 4, 6, 8), 53), _rand((2, 2, 9, 8), 54), _rand((2, 2, 9, 8), 55)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    kv = np.array([9, 4])
    for causal in (False, True):
        ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.3,
                                             enable_gqa=True).numpy()
        np.testing.assert_allclose(impl.attention(q, k, v, causal=causal, scale=0.3), ref,
                                   rtol=0, atol=1e-13)
    mask = torch.from_numpy(np.arange(9)[None, :] < kv[:, None])[:, None, None, :]
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, enable_gqa=True).numpy()
    np.testing.assert_allclose(impl.attention(q, k, v, kv_len=kv), ref, rtol=0, atol=1e-13)


# --- jagged ---------------------------------------------------------------------------

def _jagged_case(seed, lq, lk, H=4, Hkv=2, d=3):
    qo = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    ko = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    q = _rand((int(qo[-1]), H, d), seed)
    k, v = _rand((int(ko[-1]), Hkv, d), seed + 1), _rand((int(ko[-1]), Hkv, d), seed + 2)
    return q, k, v, qo, ko


def _as_dense(x):
    """One packed sequence [L, heads, d] as a one-entry dense batch [1, heads, L, d]."""
    return np.ascontiguousarray(x.transpose(1, 0, 2))[None]


def pin_jagged_brute_force(impl):
    """Each sequence of a tiny jagged batch (an empty one, one without keys, Lq != Lk,
    GQA) against the 40-digit brute force."""
    q, k, v, qo, ko = _jagged_case(60, [3, 0, 5, 2], [4, 3, 5, 0])
    for causal in (False, True):
        o = impl.attention_jagged(q, k, v, qo, ko, causal=causal, scale=0.8)
        for b in range(4):
            qs, qe, ks, ke = qo[b], qo[b + 1], ko[b], ko[b + 1]
            ref = _brute_decimal(_as_dense(q[qs:qe]), _as_dense(k[ks:ke]), _as_dense(v[ks:ke]),
                                 causal, None, 0.8)
            np.testing.assert_allclose(o[qs:qe], ref[0].transpose(1, 0, 2), rtol=0, atol=1e-12)


def pin_jagged_torch_sdpa(impl):
    """Per sequence, PyTorch's float64 SDPA (top-left causal, GQA); no keys gives zeros."""
    import torch
    import torch.nn.functional as F
    q, k, v, qo, ko = _jagged_case(63, [4, 7, 1, 3], [6, 7, 2, 0], H=4, Hkv=1, d=8)
    for causal in (False, True):
        o = impl.attention_jagged(q, k, v, qo, ko, causal=causal, scale=0.4)
        for b in range(4):
            qs, qe, ks, ke = qo[b], qo[b + 1], ko[b], ko[b + 1]
            if ke == ks:
                np.testing.assert_array_equal(o[qs:qe], 0.0)
                continue
            tq, tk, tv = (torch.from_numpy(_as_dense(x)) for x in (q[qs:qe], k[ks:ke], v[ks:ke]))
            ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.4,
                                                 enable_gqa=True).numpy()[0].transpose(1, 0, 2)
            np.testing.assert_allclose(o[qs:qe], ref, rtol=0, atol=1e-13)


def pin_jagged_equal_lengths_is_dense(impl):
    """Sequences of one common length are the dense batch in another layout."""
    B, L, H, Hkv, d = 3, 5, 4, 2, 6
    q, k, v, qo, ko = _jagged_case(66, [L] * B, [L] * B, H=H, Hkv=Hkv, d=d)
    for causal in (False, True):
        o = impl.attention_jagged(q, k, v, qo, ko, causal=causal)
        dense = impl.attention(*(x.reshape(B, L, -1, d).transpose(0, 2, 1, 3) for x in (q, k, v)),
                               causal=causal)
        np.testing.assert_allclose(o, dense.transpose(0, 2, 1, 3).reshape(B * L, H, d),
                                   rtol=0, atol=1e-14)


def pin_jagged_sequence_permutation(impl):
    """Reordering the packed sequences reorders the output the same way."""
    lq, lk = [2, 5, 3], [4, 1, 6]
    q, k, v, qo, ko = _jagged_case(69, lq, lk)
    o = impl.attention_jagged(q, k, v, qo, ko, causal=True)
    perm = [2, 0, 1]
    cat = lambda x, off: np.concatenate([x[off[b]:off[b + 1]] for b in perm])
    qo2 = np.concatenate([[0], np.cumsum([lq[b] for b in perm])])
    ko2 = np.concatenate([[0], np.cumsum([lk[b] for b in perm])])
    o2 = impl.attention_jagged(cat(q, qo), cat(k, ko), cat(v, ko), qo2, ko2, causal=True)
    np.testing.assert_array_equal(o2, cat(o, qo))


def pin_jagged_rows_subset(impl):
    """attention_jagged_rows returns exactly the matching rows of attention_jagged."""
    q, k, v, qo, ko = _jagged_case(72, [4, 6], [5, 3])
    for causal in (False, True):
        full = impl.attention_jagged(q, k, v, qo, ko, causal=causal)
        for b, rows in ((0, [3, 0]), (1, [5, 2, 1])):
            for h in (0, 3):
                part = impl.attention_jagged_rows(q, k, v, qo, ko, b, h, rows, causal=causal)
                np.testing.assert_array_equal(part, full[qo[b] + np.array(rows), h])


# --- fixed-block sparse -----------------------------------------------------------------

def _block_mask(shape, seed, density=0.6):
    m = (_rng(seed).random(shape) < density).astype(np.uint8)
    return m


def pin_block_sparse_all_ones_is_dense(impl):
    """A mask with every block set is dense attention, bit for bit."""
    q, k, v = _rand((2, 4, 9, 5), 80), _rand((2, 2, 11, 5), 81), _rand((2, 2, 11, 5), 82)
    for causal in (False, True):
        for kv in (None, np.array([11, 6])):
            o = impl.attention_block_sparse(q, k, v, np.ones((1, 3, 3), np.uint8), 4,
                                            causal=causal, kv_len=kv)
            np.testing.assert_array_equal(o, impl.attention(q, k, v, causal=causal, kv_len=kv))


def _brute_block(q, k, v, bm, blk, causal, scale):
    """40-digit direct evaluation with the block condition written out."""
    getcontext().prec = 40
    B, H, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    o = np.zeros(q.shape)
    sc = Decimal(repr(scale))
    for b in range(B):
        for h in range(H):
            g = (h * Hkv) // H
            m = bm[0] if bm.shape[0] == 1 else bm[h]
            for i in range(Lq):
                ws, num = [], [Decimal(0)] * d
                for j in range(Lk):
                    if (causal and j > i) or not m[i // blk][j // blk]:
                        continue
                    s = sum(Decimal(repr(float(q[b, h, i, t]))) * Decimal(repr(float(k[b, g, j, t])))
                            for t in range(d))
                    w = (sc * s).exp()
                    ws.append(w)
                    for t in range(d):
                        num[t] += w * Decimal(repr(float(v[b, g, j, t])))
                z = sum(ws, Decimal(0))
                if z > 0:
                    o[b, h, i] = [float(x / z) for x in num]
    return o


def pin_block_sparse_brute_force(impl):
    """Per-head masks (one query block with no key block at all), ragged edges: brute force."""
    q, k, v = _rand((1, 2, 7, 3), 83), _rand((1, 1, 6, 3), 84), _rand((1, 1, 6, 3), 85)
    bm = np.array([[[1, 0, 1], [0, 0, 0], [1, 1, 0], [0, 1, 1]],
                   [[0, 1, 0], [1, 1, 1], [0, 0, 1], [1, 0, 0]]], np.uint8)
    for causal in (False, True):
        o = impl.attention_block_sparse(q, k, v, bm, 2, causal=causal, scale=0.9)
        np.testing.assert_allclose(o, _brute_block(q, k, v, bm, 2, causal, 0.9), rtol=0,
                                   atol=1e-12)


def pin_block_sparse_is_gathered_keys(impl):
    """Without causal masking, a query block attends exactly to the keys of its set blocks:
    dense attention over those keys, gathered."""
    blk = 3
    q, k, v = _rand((1, 2, 9, 4), 86), _rand((1, 2, 12, 4), 87), _rand((1, 2, 12, 4), 88)
    bm = np.array([[[1, 0, 0, 1], [0, 1, 1, 0], [1, 1, 1, 1]]], np.uint8)
    o = impl.attention_block_sparse(q, k, v, bm, blk)
    for qb in range(3):
        keys = np.concatenate([np.arange(kb * blk, (kb + 1) * blk) for kb in range(4)
                               if bm[0, qb, kb]])
        ref = impl.attention(q[:, :, qb * blk:(qb + 1) * blk], k[:, :, keys], v[:, :, keys])
        np.testing.assert_allclose(o[:, :, qb * blk:(qb + 1) * blk], ref, rtol=0, atol=1e-14)


def pin_block_sparse_torch_sdpa(impl):
    """PyTorch's float64 SDPA with the block mask expanded to a boolean element mask."""
    import torch
    import torch.nn.functional as F
    blk, Lq, Lk = 4, 10, 14
    q, k, v = _rand((2, 4, Lq, 8), 89), _rand((2, 2, Lk, 8), 90), _rand((2, 2, Lk, 8), 91)
    bm = _block_mask((4, 3, 4), 92)
    bm[:, :, 0] = 1          # every query block keeps a block (SDPA gives NaN rows otherwise)
    for causal in (False, True):
        allow = np.kron(bm, np.ones((blk, blk), np.uint8))[:, :Lq, :Lk].astype(bool)
        if causal:
            allow &= np.tril(np.ones((Lq, Lk), bool))[None]
        ref = F.scaled_dot_product_attention(*(torch.from_numpy(x) for x in (q, k, v)),
                                             attn_mask=torch.from_numpy(allow)[None], scale=0.35,
                                             enable_gqa=True).numpy()
        o = impl.attention_block_sparse(q, k, v, bm, blk, causal=causal, scale=0.35)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)


def pin_block_sparse_shared_mask(impl):
    """One mask for all heads equals that mask repeated per head; rows subsets agree."""
    q, k, v = _rand((2, 3, 8, 4), 93), _rand((2, 3, 8, 4), 94), _rand((2, 3, 8, 4), 95)
    bm = _block_mask((1, 4, 4), 96)
    o1 = impl.attention_block_sparse(q, k, v, bm, 2, causal=True)
    o2 = impl.attention_block_sparse(q, k, v, np.repeat(bm, 3, axis=0), 2, causal=True)
    np.testing.assert_array_equal(o1, o2)
    part = impl.attention_block_sparse_rows(q, k, v, bm, 2, 1, 2, [5, 0, 3], causal=True)
    np.testing.assert_array_equal(part, o1[1, 2, [5, 0, 3]])


# --- in-kernel broadcast linear layer -------------------------------------------

def _ikbo_case(seed, B_u=3, B_c=7, K_u=5, K_c=4, N=6):
    rng = _rng(seed)
    xu = rng.standard_normal((B_u, K_u))
    xc = rng.standard_normal((B_c, K_c))
    w = rng.standard_normal((N, K_u + K_c))
    b = rng.standard_normal(N)
    c2u = rng.integers(0, B_u, B_c)
    return xu, xc, w, b, c2u


def pin_ikbo_brute_force(impl):
    """Loops over (candidate, output) on the explicitly concatenated feature vector,
    summed exactly (math.fsum), with and without a bias."""
    xu, xc, w, b, c2u = _ikbo_case(61)
    for bias in (b, None):
        y = impl.ikbo_linear(xu, xc, w, c2u, bias)
        for c in range(xc.shape[0]):
            f = list(xu[c2u[c]]) + list(xc[c])
            for n in range(w.shape[0]):
                want = math.fsum([f[t] * w[n, t] for t in range(len(f))] +
                                 ([bias[n]] if bias is not None else []))
                assert abs(y[c, n] - want) <= 1e-12, (c, n, y[c, n], want)


def pin_ikbo_torch_linear(impl):
    """torch.nn.functional.linear (float64) on the replicated, concatenated features."""
    import torch
    xu, xc, w, b, c2u = _ikbo_case(62, B_u=4, B_c=11, K_u=9, K_c=3, N=5)
    feats = torch.cat([torch.from_numpy(xu)[torch.from_numpy(c2u)], torch.from_numpy(xc)], 1)
    want = torch.nn.functional.linear(feats, torch.from_numpy(w), torch.from_numpy(b)).numpy()
    np.testing.assert_allclose(impl.ikbo_linear(xu, xc, w, c2u, b), want, rtol=0, atol=1e-12)


def pin_ikbo_permutation_weight(impl):
    """A 0/1 weight that picks feature perm[n] for output n: y[:, n] = feats[:, perm[n]],
    where the features are the user's (first K_u) and then the candidate's."""
    xu, xc, _, _, c2u = _ikbo_case(63, K_u=4, K_c=3)
    K = xu.shape[1] + xc.shape[1]
    perm = _rng(64).permutation(K)
    w = np.zeros((K, K))
    w[np.arange(K), perm] = 1.0
    y = impl.ikbo_linear(xu, xc, w, c2u)
    for c in range(xc.shape[0]):
        for n in range(K):
            t = perm[n]
            want = xu[c2u[c], t] if t < xu.shape[1] else xc[c, t - xu.shape[1]]
            assert y[c, n] == want


def pin_ikbo_same_user_rows(impl):
    """Candidates with no features of their own (x_cand = 0) get their user's row of
    the user partial; equal candidate features of one user give equal rows."""
    xu, _, w, b, c2u = _ikbo_case(65, B_c=9)
    xc = np.zeros((9, 4))
    y = impl.ikbo_linear(xu, xc, w, c2u, b)
    z = impl.ikbo_user_partial(xu, w, b)
    np.testing.assert_allclose(y, z[c2u], rtol=0, atol=1e-12)
    xc = np.tile(_rand((1, 4), 66), (9, 1))
    y = impl.ikbo_linear(xu, xc, w, np.zeros(9, np.int64), b)
    assert np.all(y == y[0])


def pin_ikbo_user_partial_brute_force(impl):
    """z[u, n] = sum over the first K_u weight columns only, plus the bias."""
    xu, _, w, b, _ = _ikbo_case(67, K_u=3, K_c=5)
    z = impl.ikbo_user_partial(xu, w, b)
    for u in range(xu.shape[0]):
        for n in range(w.shape[0]):
            want = math.fsum([xu[u, t] * w[n, t] for t in range(3)] + [b[n]])
            assert abs(z[u, n] - want) <= 1e-12


def pin_ikbo_out_of_range_user_is_nan(impl):
    """cand2user outside [0, B_u): that row is NaN, every other row is finite and
    unchanged."""
    xu, xc, w, b, c2u = _ikbo_case(68)
    bad = c2u.copy()
    bad[[1, 4]] = [-1, xu.shape[0]]
    y = impl.ikbo_linear(xu, xc, w, bad, b)
    y0 = impl.ikbo_linear(xu, xc, w, c2u, b)
    assert np.all(np.isnan(y[[1, 4]]))
    keep = [c for c in range(len(c2u)) if c not in (1, 4)]
    assert np.array_equal(y[keep], y0[keep])


def pin_ikbo_candidate_permutation(impl):
    """Permuting candidates (their features and map together) permutes the rows."""
    xu, xc, w, b, c2u = _ikbo_case(69, B_c=10)
    perm = _rng(70).permutation(10)
    y = impl.ikbo_linear(xu, xc, w, c2u, b)
    yp = impl.ikbo_linear(xu, xc[perm], w, c2u[perm], b)
    np.testing.assert_allclose(yp, y[perm], rtol=0, atol=1e-13)


# --- normalisation fused into attention ------------------------------------------

def pin_rms_norm_torch(impl):
    """torch.nn.functional.rms_norm in float64, with and without a gain, two eps."""
    import torch
    x = _rand((3, 4, 7, 16), 71)
    g = 1.0 + 0.3 * _rand((16,), 72)
    for eps in (1e-6, 0.25):
        for gamma in (g, None):
            want = torch.nn.functional.rms_norm(
                torch.from_numpy(x), (16,), None if gamma is None else torch.from_numpy(gamma),
                eps).numpy()
            np.testing.assert_allclose(impl.rms_norm(x, gamma, eps), want, rtol=0, atol=1e-13)


def pin_rms_norm_closed_forms(impl):
    """eps = 0: a constant row c becomes sign(c) * gamma; a one-hot row a e_t becomes
    sign(a) sqrt(d) e_t * gamma; a zero row stays zero for eps > 0."""
    d = 8
    g = np.arange(1, d + 1, dtype=float)
    for c in (3.0, -0.5):
        np.testing.assert_allclose(impl.rms_norm(np.full((1, d), c), g, 0.0)[0], np.sign(c) * g,
                                   rtol=1e-15, atol=0)
    x = np.zeros((1, d))
    x[0, 5] = -2.5
    want = np.zeros(d)
    want[5] = -math.sqrt(d) * g[5]
    np.testing.assert_allclose(impl.rms_norm(x, g, 0.0)[0], want, rtol=1e-15, atol=0)
    assert np.all(impl.rms_norm(np.zeros((2, d)), g, 1e-6) == 0)


def pin_qknorm_torch_sdpa(impl):
    """torch float64 SDPA (GQA, causal, kv_len mask) on rows normalised by torch's
    rms_norm with the query gain on q and the key gain on k; v as given."""
    import torch
    F = torch.nn.functional
    B, H, Hkv, Lq, Lk, d = 2, 4, 2, 9, 11, 8
    q, k, v = (torch.from_numpy(_rand(s, 73 + i)) for i, s in
               enumerate([(B, H, Lq, d), (B, Hkv, Lk, d), (B, Hkv, Lk, d)]))
    gq, gk = (torch.from_numpy(1.0 + 0.3 * _rand((d,), 80 + i)) for i in range(2))
    kv_len = np.array([11, 6])
    eps = 1e-3
    qn, kn = F.rms_norm(q, (d,), gq, eps), F.rms_norm(k, (d,), gk, eps)
    mask = torch.arange(Lk)[None, :] < torch.from_numpy(kv_len)[:, None]
    causal = torch.ones(Lq, Lk, dtype=torch.bool).tril()
    attn_mask = mask[:, None, None, :] & causal[None, None]
    want = F.scaled_dot_product_attention(qn, kn, v, attn_mask=attn_mask,
                                          enable_gqa=True).numpy()
    got = impl.attention_qknorm(q.numpy(), k.numpy(), v.numpy(), gq.numpy(), gk.numpy(), eps,
                                causal=True, kv_len=kv_len)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def pin_qknorm_row_scale_invariance(impl):
    """With eps = 0, scaling any query or key row by a positive factor changes nothing,
    while scaling v scales the output."""
    q, k, v = _rand((1, 2, 6, 8), 91), _rand((1, 2, 7, 8), 92), _rand((1, 2, 7, 8), 93)
    a = np.exp(_rand((1, 2, 6, 1), 94))
    b = np.exp(_rand((1, 2, 7, 1), 95))
    o = impl.attention_qknorm(q, k, v, None, None, 0.0, causal=True)
    np.testing.assert_allclose(impl.attention_qknorm(q * a, k * b, v, None, None, 0.0,
                                                     causal=True), o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(impl.attention_qknorm(q, k, 3.0 * v, None, None, 0.0,
                                                     causal=True), 3.0 * o, rtol=0, atol=1e-12)


def pin_qknorm_rows(impl):
    """attention_qknorm_rows equals the same rows of attention_qknorm."""
    q, k, v = _rand((2, 4, 9, 8), 96), _rand((2, 2, 10, 8), 97), _rand((2, 2, 10, 8), 98)
    gq, gk = 1.0 + 0.2 * _rand((8,), 99), 1.0 + 0.2 * _rand((8,), 100)
    full = impl.attention_qknorm(q, k, v, gq, gk, 1e-5, causal=True, kv_len=np.array([10, 4]))
    rows = np.array([0, 3, 8])
    got = impl.attention_qknorm_rows(q, k, v, 1, 3, rows, gq, gk, 1e-5, causal=True,
                                     kv_len=np.array([10, 4]))
    np.testing.assert_allclose(got, full[1, 3, rows], rtol=0, atol=1e-14)


ALL_PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_")]
