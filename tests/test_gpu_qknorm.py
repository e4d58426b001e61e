"""Attention on RMS-normalised queries and keys on the GPU against the float64
oracle, element by element, through the C ABI; the key workspace against the
oracle's normalised keys."""
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


def run(taa, w):
    import torch
    q, k, v = (to_dev(x, "bf16") for x in (w.q, w.k, w.v))
    gq = None if w.gamma_q is None else torch.from_numpy(w.gamma_q).cuda()
    gk = None if w.gamma_k is None else torch.from_numpy(w.gamma_k).cuda()
    kn = torch.empty_like(k)
    o = taa.attn_fwd_qknorm(q, k, v, gq, gk, w.eps, k_norm=kn, causal=w.causal,
                            kv_len=i32_dev(w.kv_len), scale=w.scale or 0.0)
    torch.cuda.synchronize()
    return from_dev(o), from_dev(kn)


def ref(w):
    q, k, v = w.f64()
    return oracle.attention_qknorm(q, k, v, w.gamma_q, w.gamma_k, w.eps, causal=w.causal,
                                   kv_len=w.kv_len, scale=w.scale)


QKNORM_CASES = [
    # (B, H, Hkv, Lq, Lk, d, causal, kv_len range, gains, eps)
    (1, 4, 2, 300, 300, 128, True, None, True, 1e-6),
    (2, 2, 2, 200, 333, 64, False, (100, 333), True, 1e-6),
    (1, 2, 1, 4500, 4600, 128, True, None, True, 1e-6),        # 8-wave schedule
    (1, 2, 2, 128, 128, 128, False, None, False, 1e-6),        # no gains
    (1, 2, 2, 70, 90, 64, True, None, True, 0.5),              # eps matters
]


def _random_qknorm_cases(n=4, seed=2030):
    """Seeded q/k-normalised problems in small ranges, both head dims."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        Hkv = int(rng.integers(1, 3))
        Lk = int(rng.integers(1, 500))
        kvr = (int(rng.integers(0, Lk)), Lk) if rng.random() < 0.4 else None
        cases.append((int(rng.integers(1, 3)), Hkv * int(rng.choice([1, 2, 4])), Hkv,
                      int(rng.integers(1, 400)), Lk, int(rng.choice([64, 128])),
                      bool(rng.random() < 0.5), kvr, bool(rng.random() < 0.7), 1e-6))
    return cases


QKNORM_CASES += _random_qknorm_cases()


@pytest.mark.parametrize("case", QKNORM_CASES,
                         ids=lambda c: f"d{c[5]}-c{int(c[6])}-L{c[3]}x{c[4]}-g{int(c[8])}-e{c[9]}")
def test_qknorm_matches_oracle(lib, case):
    B, H, Hkv, Lq, Lk, d, causal, kvr, gains, eps = case
    w = ai.make_qknorm(B, H, Hkv, Lq, Lk, d, causal=causal, seed=51, kv_len_range=kvr, eps=eps,
                       gains=gains)
    got, kn = run(lib, w)
    assert max_err(got, ref(w)) <= TOL["bf16"]
    # the key workspace: normalised keys, rounded once to bf16
    want = oracle.rms_norm(ai.to_f64(w.k, "bf16"), w.gamma_k, eps)
    assert np.all(np.abs(kn - want) <= 2.0 ** -8 * np.abs(want) * (1 + 1e-5) + 1e-30)


def test_qknorm_differs_from_plain_attention(lib):
    """The inputs make normalisation matter: plain attention is far from the result."""
    w = ai.make_qknorm(1, 2, 2, 200, 200, 128, causal=True, seed=53)
    got, _ = run(lib, w)
    q, k, v = w.f64()
    assert max_err(got, oracle.attention(q, k, v, causal=True)) > 0.1
    assert max_err(got, ref(w)) <= TOL["bf16"]


def test_qknorm_without_keys_gives_zeros(lib):
    import torch
    w = ai.make_qknorm(1, 2, 2, 64, 1, 64, seed=55)
    q = to_dev(w.q, "bf16")
    k = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    o = lib.attn_fwd_qknorm(q, k, k, k_norm=torch.empty_like(k))
    torch.cuda.synchronize()
    assert np.all(from_dev(o) == 0)


def test_qknorm_full_size_workload_sampled(lib):
    import torch
    w = ai.make_workload("qknorm_gqa_causal_L16384", seed=0)
    q, k, v = (to_dev(x, "bf16") for x in (w.q, w.k, w.v))
    o = nan_filled(q)
    lib.attn_fwd_qknorm(q, k, v, torch.from_numpy(w.gamma_q).cuda(),
                        torch.from_numpy(w.gamma_k).cuda(), w.eps, o, causal=w.causal)
    torch.cuda.synchronize()
    assert_all_written(o)
    rng = np.random.default_rng(17)
    B, H, Lq, _ = w.q.shape
    worst = 0.0
    qf, kf, vf = w.f64()
    for h in [0, H - 1, int(rng.integers(H))]:
        rows = np.unique(np.concatenate([[0, 1, 4095, 4096, Lq - 1], rng.integers(0, Lq, 8)]))
        got = o[0, h, torch.from_numpy(rows).cuda()].to(torch.float64).cpu().numpy()
        want = oracle.attention_qknorm_rows(qf, kf, vf, 0, h, rows, w.gamma_q, w.gamma_k, w.eps,
                                            causal=w.causal)
        worst = max(worst, max_err(got, want))
    assert worst <= TOL["bf16"], worst
