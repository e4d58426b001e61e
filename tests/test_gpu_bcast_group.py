"""Candidate grouping for the broadcast attention (attn_bcast_group) and the
broadcast attention with a packing order (attn_fwd_bcast_grouped).

The grouping is a counting sort by user on the device: checked here for being
a permutation in which each user's candidates form one run, users in
increasing order and out-of-range users last. The attention with any packing
order computes every candidate with the same arithmetic, so its output must
equal attn_fwd_bcast's bit for bit (and the oracle within the bf16 bound).
"""
import numpy as np
import pytest

import attn_inputs as ai
import oracle
from gpu_util import TOL, from_dev, i32_dev, max_err, nan_filled, assert_all_written, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tiled_attention_attn_amd as taa
    taa.load_library()
    return taa


def _bucket(c2u, B_u):
    return np.where((c2u >= 0) & (c2u < B_u), c2u, B_u)


@pytest.mark.parametrize("B_c,B_u,bad", [
    (1, 1, 0), (7, 3, 0), (1024, 32, 0), (1024, 32, 9), (3000, 5, 40),   # several passes per thread
    (5000, 2500, 17),   # more buckets than threads: the offset scan runs in chunks
    (64, 4096, 3),      # most users have no candidate
])
def test_group_is_a_grouped_permutation(lib, B_c, B_u, bad):
    import torch
    rng = np.random.default_rng(B_c * 7 + B_u)
    c2u = rng.integers(0, B_u, size=B_c).astype(np.int32)
    if bad:
        idx = rng.choice(B_c, size=bad, replace=False)
        c2u[idx] = rng.choice([-1, -1000, B_u, B_u + 5, 1 << 30], size=bad)
    order = lib.bcast_group(i32_dev(c2u), B_u).cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(np.sort(order), np.arange(B_c)), "not a permutation"
    b = _bucket(c2u, B_u)[order]
    assert np.all(np.diff(b) >= 0), "users not grouped in increasing order"
    # each user's run holds exactly its candidates
    for u in np.unique(b)[:50]:
        assert set(order[b == u]) == set(np.flatnonzero(_bucket(c2u, B_u) == u))


def test_group_twice_on_one_workspace(lib):
    """The workspace is rewritten from zero on every call."""
    import torch
    B_c, B_u = 500, 9
    c2u = np.random.default_rng(5).integers(0, B_u, size=B_c).astype(np.int32)
    d = i32_dev(c2u)
    o1 = lib.bcast_group(d, B_u).cpu().numpy()
    o2 = lib.bcast_group(d, B_u).cpu().numpy()
    torch.cuda.synchronize()
    for o in (o1, o2):
        assert np.array_equal(np.sort(o), np.arange(B_c))
        assert np.all(np.diff(c2u[o]) >= 0)


GROUPED_CASES = [
    # (B_c, B_u, H, Hkv, Lq, Lk, d, dtype, causal)
    (64, 5, 2, 2, 64, 300, 128, "bf16", False),    # 2 candidates per 4-wave workgroup
    (64, 5, 2, 1, 32, 200, 128, "bf16", True),     # 4 per workgroup
    (48, 7, 2, 2, 20, 150, 64, "bf16", False),     # 4 per workgroup, d = 64
    (30, 4, 2, 2, 100, 130, 128, "bf16", True),    # one per workgroup: order only permutes
    (16, 3, 2, 2, 64, 4200, 128, "bf16", False),   # 8-wave schedule: 4 per workgroup
    (20, 3, 2, 2, 50, 60, 64, "f32", False),       # fp32 path: the order is ignored
]


@pytest.mark.parametrize("case", GROUPED_CASES, ids=lambda c: "-".join(map(str, c)))
def test_grouped_equals_ungrouped_and_oracle(lib, case):
    import torch
    B_c, B_u, H, Hkv, Lq, Lk, d, dtype, causal = case
    rng = np.random.default_rng(B_c + Lq)
    c2u = rng.integers(0, B_u, size=B_c).astype(np.int32)
    c2u[[1, B_c // 2]] = [-1, B_u]          # two bad users: NaN rows either way
    w = ai.make_bcast(B_c, B_u, H, Hkv, Lq, Lk, d, dtype=dtype, causal=causal, seed=71,
                      cand2user=c2u, kv_len_range=(1, Lk))
    q, k, v = (to_dev(x, dtype) for x in (w.q, w.k, w.v))
    cu, kl = i32_dev(c2u), i32_dev(w.kv_len)
    plain = lib.attn_fwd_bcast(q, k, v, cu, causal=causal, kv_len=kl)
    order = lib.bcast_group(cu, B_u)
    o = nan_filled(q)
    lib.attn_fwd_bcast(q, k, v, cu, o, causal=causal, kv_len=kl, order=order)
    torch.cuda.synchronize()
    got, want = from_dev(o), from_dev(plain)
    assert np.array_equal(got, want, equal_nan=True)
    good = np.flatnonzero((c2u >= 0) & (c2u < B_u))
    assert np.all(np.isnan(got[[1, B_c // 2]]))
    qf, kf, vf = w.f64()
    ref = oracle.attention_bcast(qf, kf, vf, c2u, causal=causal, kv_len=w.kv_len)
    assert max_err(got[good], ref[good]) <= TOL[dtype]


def test_grouped_any_permutation_and_full_write(lib):
    """A random packing order (not grouped) is still exact, and every row is written."""
    import torch
    B_c, B_u = 40, 6
    c2u = np.random.default_rng(3).integers(0, B_u, size=B_c).astype(np.int32)
    w = ai.make_bcast(B_c, B_u, 2, 2, 64, 180, 128, seed=72, cand2user=c2u)
    q, k, v = (to_dev(x, "bf16") for x in (w.q, w.k, w.v))
    cu = i32_dev(c2u)
    plain = lib.attn_fwd_bcast(q, k, v, cu)
    perm = i32_dev(np.random.default_rng(4).permutation(B_c).astype(np.int32))
    o = nan_filled(q)
    lib.attn_fwd_bcast(q, k, v, cu, o, order=perm)
    torch.cuda.synchronize()
    assert_all_written(o)
    assert torch.equal(o.view(torch.int16), plain.view(torch.int16))
