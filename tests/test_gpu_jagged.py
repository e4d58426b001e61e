"""Jagged attention (packed sequences with offsets) on the GPU against the
float64 oracle, element by element, through the C ABI."""
import numpy as np
import pytest

import attn_inputs as ai
import oracle
from gpu_util import TOL, assert_all_written, from_dev, i32_dev, max_err, nan_filled, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tiled_attention_attn_amd as taa
    taa.load_library()
    return taa


def run_jagged(taa, w, max_lq=None, max_lk=None, o=None):
    import torch
    q, k, v = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v))
    out = taa.attn_fwd_jagged(q, k, v, i32_dev(w.q_offsets), i32_dev(w.kv_offsets),
                              w.meta["max_Lq"] if max_lq is None else max_lq,
                              w.meta["max_Lk"] if max_lk is None else max_lk, o,
                              causal=w.causal, scale=w.scale or 0.0)
    torch.cuda.synchronize()
    return from_dev(out)


def ref_jagged(w):
    q, k, v = w.f64()
    return oracle.attention_jagged(q, k, v, w.q_offsets, w.kv_offsets, causal=w.causal,
                                   scale=w.scale)


JAGGED_CASES = [
    # (H, Hkv, d, dtype, causal, query lengths, key lengths or None = same)
    (2, 2, 128, "bf16", True, [100, 0, 257, 64, 1], None),
    (4, 2, 128, "bf16", False, [300, 77, 130], [129, 0, 500]),    # Lq != Lk, one without keys
    (2, 1, 64, "bf16", True, [33, 200, 513], [80, 150, 513]),     # causal top-left, Lq != Lk
    (3, 3, 128, "bf16", False, [20, 40, 7, 64, 10, 33], None),    # short: several per workgroup
    (2, 2, 64, "f32", True, [70, 0, 129], None),
    (2, 1, 128, "f32", False, [40, 90], [60, 0]),
    (2, 2, 128, "bf16", True, [8300, 500], None),                 # 8-wave schedule
    (2, 1, 128, "bf16", False, [700, 64], [8250, 9000]),
]


def _random_jagged_cases(n=6, seed=2028):
    """Seeded packed batches: 1-7 sequences of 0-600 tokens (keys the same lengths or
    drawn apart), both head dims, GQA or not, causal or not."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        Hkv = int(rng.integers(1, 3))
        nb = int(rng.integers(1, 8))
        lq = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 600, size=nb)]
        lk = None if rng.random() < 0.5 else [int(x) for x in rng.integers(0, 600, size=nb)]
        cases.append((Hkv * int(rng.choice([1, 2])), Hkv, int(rng.choice([64, 128])), "bf16",
                      bool(rng.random() < 0.5), lq, lk))
    return cases


JAGGED_CASES += _random_jagged_cases()


@pytest.mark.parametrize("case", JAGGED_CASES, ids=lambda c: f"{c[3]}-d{c[2]}-c{int(c[4])}-"
                         f"{'_'.join(map(str, c[5]))}")
def test_jagged_matches_oracle(lib, case):
    H, Hkv, d, dtype, causal, lq, lk = case
    w = ai.make_jagged(len(lq), H, Hkv, d, lengths=lq, kv_lengths=lk, dtype=dtype,
                       causal=causal, seed=17)
    got = run_jagged(lib, w)
    want = ref_jagged(w)
    assert max_err(got, want) <= TOL[dtype]
    for b in range(len(lq)):   # sequences without keys give exact zero rows
        if w.kv_offsets[b + 1] == w.kv_offsets[b]:
            assert np.all(got[w.q_offsets[b]:w.q_offsets[b + 1]] == 0)


def test_jagged_equal_lengths_match_dense_kernel(lib):
    """Equal lengths: the jagged call and the dense call on the transposed layout agree
    to rounding (their tile decompositions differ only in addressing)."""
    import torch
    B, L, H, d = 3, 200, 2, 128
    w = ai.make_jagged(B, H, H, d, lengths=[L] * B, causal=True, seed=19)
    got = run_jagged(lib, w)
    q, k, v = (to_dev(x, "bf16").reshape(B, L, H, d).transpose(1, 2).contiguous()
               for x in (w.q, w.k, w.v))
    o = lib.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    dense = from_dev(o.transpose(1, 2).reshape(B * L, H, d))
    assert np.array_equal(got, dense)


def test_jagged_lengths_past_max_are_cut(lib):
    """Rows past max_lq are not written; keys past max_lk are ignored."""
    import torch
    w = ai.make_jagged(2, 2, 2, 64, lengths=[100, 50], causal=False, seed=23)
    sentinel = 7.0
    o = torch.full(w.q.shape, sentinel, dtype=torch.bfloat16, device="cuda")
    got = run_jagged(lib, w, max_lq=80, max_lk=60, o=o)
    q, k, v = w.f64()
    want0 = oracle.attention_jagged(q[:80], k[:60], v[:60], [0, 80], [0, 60])
    want1 = oracle.attention_jagged(q[100:], k[100:], v[100:], [0, 50], [0, 50])
    assert max_err(got[:80], want0) <= TOL["bf16"]
    assert np.all(got[80:100] == sentinel)
    assert max_err(got[100:], want1) <= TOL["bf16"]


def test_jagged_full_size_workload_sampled(lib):
    import torch
    w = ai.make_workload("jagged_causal_B32", seed=0)
    q, k, v = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v))
    o = nan_filled(q)
    lib.attn_fwd_jagged(q, k, v, i32_dev(w.q_offsets), i32_dev(w.kv_offsets),
                        w.meta["max_Lq"], w.meta["max_Lk"], o, causal=w.causal)
    torch.cuda.synchronize()
    assert_all_written(o)
    rng = np.random.default_rng(9)
    B, H, Hkv = len(w.q_offsets) - 1, w.q.shape[1], w.k.shape[1]
    worst = 0.0
    for b, h in [(0, 0), (B - 1, H - 1)] + [(int(rng.integers(B)), int(rng.integers(H)))
                                            for _ in range(4)]:
        qs, qe = int(w.q_offsets[b]), int(w.q_offsets[b + 1])
        ks, ke = int(w.kv_offsets[b]), int(w.kv_offsets[b + 1])
        L = qe - qs
        rows = np.unique(np.concatenate([[0, 1, 63, 64, L // 2, L - 1], rng.integers(0, L, 6)]))
        got = o[torch.from_numpy(qs + rows).cuda(), h].to(torch.float64).cpu().numpy()
        g = h // (H // Hkv)
        ref = oracle.attention_jagged_rows(
            ai.to_f64(w.q[qs:qe, h:h + 1], w.dtype), ai.to_f64(w.k[ks:ke, g:g + 1], w.dtype),
            ai.to_f64(w.v[ks:ke, g:g + 1], w.dtype), [0, L], [0, ke - ks], 0, 0, rows,
            causal=w.causal)
        worst = max(worst, max_err(got, ref))
    assert worst <= TOL[w.dtype], worst
