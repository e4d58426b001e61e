"""HIP path against the float64 oracle, element by element, through the C ABI.

Small cases cover several tiles, ragged tails, every mask kind, GQA, the
query-packing modes of short sequences, and the broadcast variant. The
full-size workloads are checked on sampled rows the oracle computes one by one.
"""
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


def run_dense(taa, w):
    import torch
    q, k, v = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v))
    o = taa.attn_fwd(q, k, v, causal=w.causal, kv_len=i32_dev(w.kv_len), scale=w.scale or 0.0)
    torch.cuda.synchronize()
    return from_dev(o)


def run_bcast(taa, w, cand2user=None):
    import torch
    q, k, v = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v))
    c2u = w.cand2user if cand2user is None else cand2user
    o = taa.attn_fwd_bcast(q, k, v, i32_dev(c2u), causal=w.causal, kv_len=i32_dev(w.kv_len),
                           scale=w.scale or 0.0)
    torch.cuda.synchronize()
    return from_dev(o)


def ref_dense(w):
    q, k, v = w.f64()
    return oracle.attention(q, k, v, causal=w.causal, kv_len=w.kv_len, scale=w.scale)


DENSE_CASES = [
    # (B, H, Hkv, Lq, Lk, d, dtype, causal, kv_len_range)
    (1, 1, 1, 128, 128, 64, "f32", False, None),        # the tiny fp32 workload
    (2, 2, 1, 77, 130, 128, "f32", True, None),
    (2, 2, 2, 100, 150, 64, "f32", False, (1, 150)),
    (2, 4, 4, 300, 300, 128, "bf16", False, None),
    (2, 4, 4, 300, 300, 128, "bf16", True, None),
    (2, 2, 2, 200, 333, 64, "bf16", False, (100, 333)),
    (2, 2, 2, 333, 200, 64, "bf16", True, (1, 200)),
    (1, 8, 2, 257, 257, 128, "bf16", True, None),       # GQA 4:1
    (1, 6, 3, 129, 64, 128, "bf16", False, None),       # GQA 2:1, one key tile
    (1, 2, 2, 100, 300, 128, "bf16", True, None),       # Lq < Lk causal (top-left)
    (1, 2, 2, 300, 100, 128, "bf16", True, None),       # Lq > Lk causal
    (3, 2, 2, 64, 190, 128, "bf16", False, None),       # two entries per workgroup
    (5, 2, 1, 32, 100, 64, "bf16", True, None),         # four entries per workgroup
    (3, 2, 2, 40, 70, 128, "bf16", False, (1, 70)),     # ragged short rows
    (2, 2, 2, 96, 96, 128, "bf16", True, None),         # three row blocks, padded
    (3, 2, 2, 1, 50, 64, "bf16", False, None),          # single query row
    (1, 1, 1, 513, 1025, 128, "bf16", False, None),
    (1, 1, 1, 700, 1500, 64, "bf16", True, (1000, 1500)),
    # d=128 with Lk >= 4096 runs the 8-wave schedule
    (1, 2, 2, 300, 8200, 128, "bf16", False, None),
    (1, 4, 2, 257, 8193, 128, "bf16", True, None),
    (1, 2, 1, 100, 9000, 128, "bf16", False, (5000, 9000)),
    (1, 1, 1, 8262, 8262, 128, "bf16", True, None),
    (3, 2, 2, 64, 8250, 128, "bf16", False, None),
    (1, 2, 2, 4096, 4096, 128, "bf16", True, None),
    (2, 3, 1, 1000, 4100, 128, "bf16", True, (3000, 4100)),
    # causal with many heads per XCD chunk: row blocks ordered across heads
    (3, 6, 2, 700, 700, 128, "bf16", True, None),
    (5, 4, 4, 260, 260, 64, "bf16", True, None),
]


def _random_dense_cases(n_short=24, n_long=4, seed=2026):
    """Seeded shapes beyond the hand-picked ones: any (B, H, Hkv, Lq, Lk) in small
    ranges, both head dims, both mask kinds, a few fp32; and some d=128 problems with
    Lk >= 4096 (the 8-wave schedule), kept short in Lq for the oracle's sake."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_short + n_long):
        long = i >= n_short
        Hkv = int(rng.integers(1, 4))
        H = Hkv * int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 4))
        d = 128 if long else int(rng.choice([64, 128]))
        Lq = int(rng.integers(1, 120 if long else 400))
        Lk = int(rng.integers(4096, 6000)) if long else int(rng.integers(1, 600))
        dtype = "f32" if (not long and rng.random() < 0.2) else "bf16"
        causal = bool(rng.random() < 0.5)
        if long:
            causal = bool(i % 2)   # half of them run the whole key range
        kvr = (int(rng.integers(0, Lk)), Lk) if rng.random() < 0.4 else None
        cases.append((B, H, Hkv, Lq, Lk, d, dtype, causal, kvr))
    return cases


@pytest.mark.parametrize("case", DENSE_CASES + _random_dense_cases(),
                         ids=lambda c: "-".join(map(str, c[:8])))
def test_dense_matches_oracle(lib, case):
    B, H, Hkv, Lq, Lk, d, dtype, causal, kvr = case
    w = ai.make_dense(B, H, Hkv, Lq, Lk, d, dtype=dtype, causal=causal, seed=11,
                      kv_len_range=kvr)
    err = max_err(run_dense(lib, w), ref_dense(w))
    assert err <= TOL[dtype], f"max abs err {err}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_custom_scale(lib, dtype, d):
    w = ai.make_dense(1, 2, 2, 70, 90, d, dtype=dtype, seed=3, scale=0.05)
    err = max_err(run_dense(lib, w), ref_dense(w))
    assert err <= TOL[dtype]


def test_masked_rows_and_empty_keys_are_zero(lib):
    w = ai.make_dense(3, 2, 2, 50, 80, 128, seed=4)
    w.kv_len = np.array([0, 80, 0], dtype=np.int32)
    got = run_dense(lib, w)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert max_err(got, ref_dense(w)) <= TOL["bf16"]
    w0 = ai.make_dense(1, 2, 2, 40, 0, 64, seed=4)       # Lk = 0
    assert np.all(run_dense(lib, w0) == 0)


def test_out_of_range_kv_len_is_clamped(lib):
    w = ai.make_dense(2, 2, 2, 60, 90, 64, seed=5)
    w.kv_len = np.array([-5, 1000], dtype=np.int32)
    got = run_dense(lib, w)
    assert np.all(got[0] == 0)
    assert max_err(got, ref_dense(w)) <= TOL["bf16"]


def test_empty_problem_is_noop(lib):
    import torch
    q = torch.zeros((0, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((0, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    o = lib.attn_fwd(q, k, k)
    assert o.shape == q.shape


def test_deterministic(lib):
    import torch
    w = ai.make_dense(2, 4, 2, 300, 300, 128, causal=True, seed=6)
    q, k, v = (to_dev(x, "bf16") for x in (w.q, w.k, w.v))
    a = lib.attn_fwd(q, k, v, causal=True)
    b = lib.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# --- broadcast ------------------------------------------------------------------

BCAST_CASES = [
    # (B_c, B_u, H, Hkv, Lq, Lk, d, dtype, causal, map)
    (12, 3, 2, 2, 64, 200, 128, "bf16", False, "contiguous"),
    (12, 3, 2, 2, 64, 200, 128, "bf16", False, "shuffled"),
    (10, 4, 4, 2, 32, 150, 64, "bf16", True, "shuffled"),
    (7, 2, 2, 2, 200, 130, 128, "bf16", True, "contiguous"),
    (9, 3, 2, 1, 40, 77, 64, "bf16", False, "shuffled"),
    (6, 2, 2, 2, 50, 60, 64, "f32", False, "shuffled"),
    (8, 2, 2, 2, 64, 8200, 128, "bf16", False, "shuffled"),   # 8-wave schedule
    (5, 2, 4, 2, 40, 8300, 128, "bf16", True, "contiguous"),
]


def _random_bcast_cases(n=10, seed=2027):
    """Seeded broadcast shapes: any candidate and user counts, query and key lengths
    in small ranges, both head dims, contiguous or shuffled maps."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        Hkv = int(rng.integers(1, 3))
        H = Hkv * int(rng.choice([1, 2]))
        B_u = int(rng.integers(1, 6))
        B_c = int(rng.integers(1, 21))
        d = int(rng.choice([64, 128]))
        cases.append((B_c, B_u, H, Hkv, int(rng.integers(1, 130)), int(rng.integers(1, 400)), d,
                      "bf16", bool(rng.random() < 0.5),
                      "shuffled" if rng.random() < 0.5 else "contiguous"))
    return cases


BCAST_CASES += _random_bcast_cases()


def _map(kind, B_c, B_u, seed=0):
    if kind == "contiguous":
        return np.minimum(np.arange(B_c) // max(1, B_c // B_u), B_u - 1).astype(np.int32)
    return np.random.default_rng(seed).integers(0, B_u, size=B_c).astype(np.int32)


@pytest.mark.parametrize("case", BCAST_CASES, ids=lambda c: "-".join(map(str, c)))
def test_bcast_matches_oracle(lib, case):
    B_c, B_u, H, Hkv, Lq, Lk, d, dtype, causal, kind = case
    w = ai.make_bcast(B_c, B_u, H, Hkv, Lq, Lk, d, dtype=dtype, causal=causal, seed=12,
                      cand2user=_map(kind, B_c, B_u), kv_len_range=(1, Lk))
    q, k, v = w.f64()
    ref = oracle.attention_bcast(q, k, v, w.cand2user, causal=causal, kv_len=w.kv_len)
    err = max_err(run_bcast(lib, w), ref)
    assert err <= TOL[dtype], f"max abs err {err}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bcast_bit_equal_to_dense_on_replicated_kv(lib, dtype):
    import torch
    B_c, B_u = 16, 5
    w = ai.make_bcast(B_c, B_u, 4, 2, 64, 180, 128 if dtype == "bf16" else 64, dtype=dtype,
                      seed=13, cand2user=_map("shuffled", B_c, B_u, 1), kv_len_range=(50, 180))
    got = run_bcast(lib, w)
    rep = ai.AttnInputs(w.q, w.k[w.cand2user], w.v[w.cand2user], dtype,
                        kv_len=w.kv_len[w.cand2user])
    dense = run_dense(lib, rep)
    assert np.array_equal(got, dense)


def test_bcast_bad_user_gives_nan_rows(lib):
    w = ai.make_bcast(6, 2, 2, 2, 64, 70, 128, seed=14)
    c2u = np.array([0, 1, 2, -1, 1, 0], dtype=np.int32)
    got = run_bcast(lib, w, c2u)
    assert np.all(np.isnan(got[2])) and np.all(np.isnan(got[3]))
    good = [0, 1, 4, 5]
    q, k, v = w.f64()
    ref = oracle.attention_bcast(q, k, v, c2u)
    assert max_err(got[good], ref[good]) <= TOL["bf16"]


# --- full-size workloads on sampled rows ---------------------------------------------------

def _sample_rows(Lq, rng, n=6):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, Lq // 2, Lq - 2, Lq - 1]
    return np.unique(np.concatenate([[r for r in fixed if 0 <= r < Lq],
                                     rng.integers(0, Lq, size=n)]))


@pytest.mark.parametrize("name", ["fp32_tiny", "dense_causal_L2048", "masked_kvlen_L4096_d64",
                                  "gqa_causal_L16384", "bcast_Bc1024_Bu32"])
def test_full_size_workload_sampled(lib, name):
    import torch
    w = ai.make_workload(name, seed=0)
    dtype = w.dtype
    q, k, v = (to_dev(x, dtype) for x in (w.q, w.k, w.v))
    o = nan_filled(q)
    if w.cand2user is not None:
        lib.attn_fwd_bcast(q, k, v, i32_dev(w.cand2user), o, causal=w.causal,
                           kv_len=i32_dev(w.kv_len))
    else:
        lib.attn_fwd(q, k, v, o, causal=w.causal, kv_len=i32_dev(w.kv_len))
    torch.cuda.synchronize()
    assert_all_written(o, name)
    rng = np.random.default_rng(7)
    NB, H, Lq, d = w.q.shape
    worst = 0.0
    picks = [(0, 0), (NB - 1, H - 1)] + [(int(rng.integers(NB)), int(rng.integers(H)))
                                         for _ in range(4)]
    for b, h in picks:
        rows = _sample_rows(Lq, rng)
        got = o[b, h, torch.from_numpy(rows).cuda()].to(torch.float64).cpu().numpy()
        qf = ai.to_f64(w.q[b:b + 1, h:h + 1], dtype)
        if w.cand2user is not None:
            u = int(w.cand2user[b])
            kf, vf = ai.to_f64(w.k[u:u + 1], dtype), ai.to_f64(w.v[u:u + 1], dtype)
            kvl = None if w.kv_len is None else w.kv_len[u:u + 1]
            g = h // (H // w.k.shape[1])
        else:
            kf, vf = ai.to_f64(w.k[b:b + 1], dtype), ai.to_f64(w.v[b:b + 1], dtype)
            kvl = None if w.kv_len is None else w.kv_len[b:b + 1]
            g = h // (H // w.k.shape[1])
        ref = oracle.attention_rows(qf, kf[:, g:g + 1], vf[:, g:g + 1], 0, 0, rows,
                                    causal=w.causal, kv_len=kvl)
        worst = max(worst, max_err(got, ref))
    assert worst <= TOL[dtype], f"{name}: max abs err {worst}"


@pytest.mark.parametrize("d,causal", [(128, True), (128, False), (64, False)])
def test_both_schedules_agree_with_oracle(lib, d, causal, tmp_path):
    """Force each wave schedule (child processes with ATTN_BF16_WAVES) on the same inputs;
    both match the oracle."""
    import subprocess
    import sys
    w = ai.make_dense(2, 4, 2, 300, 700, d, causal=causal, seed=21, kv_len_range=(400, 700))
    ref = ref_dense(w)
    np.savez(tmp_path / "in.npz", q=w.q, k=w.k, v=w.v, kv_len=w.kv_len)
    script = (
        "import sys, numpy as np, torch; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
        "import tiled_attention_attn_amd as taa; from gpu_util import to_dev, from_dev, i32_dev\n"
        "z = np.load(%r)\n"
        "o = taa.attn_fwd(*(to_dev(z[n], 'bf16') for n in 'qkv'), causal=%r, kv_len=i32_dev(z['kv_len']))\n"
        "torch.cuda.synchronize(); np.save(%r, from_dev(o))\n"
    )
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = {}
    for waves in ("4", "8"):
        out = tmp_path / f"o{waves}.npy"
        env = dict(os.environ, ATTN_BF16_WAVES=waves)
        code = script % (root, os.path.join(root, "tests"), str(tmp_path / "in.npz"), causal, str(out))
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                           timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        outs[waves] = np.load(out)
        assert max_err(outs[waves], ref) <= TOL["bf16"], waves
    # the schedules keep the softmax reference differently: equal up to rounding
    assert max_err(outs["4"], outs["8"]) <= TOL["bf16"]


_MOVES = [(1000, 64, False, "bf16"), (1000, 128, True, "bf16"), (8192, 128, False, "bf16"),
          (8192, 128, True, "bf16")]


@pytest.mark.parametrize("Lk,d,causal,dtype,growth",
                         [c + (g,) for c in _MOVES for g in (12.0, 80.0)]
                         + [(700, 64, False, "f32", 12.0), (700, 128, True, "f32", 12.0)],
                         ids=lambda v: str(v))
def test_reference_moves_on_every_tile(lib, Lk, d, causal, dtype, growth):
    """Keys along the query direction, scaled up with the key index: each 64-key tile raises
    every row's maximum by `growth` (in base 2, after the softmax scale) over the last one,
    past the 2^8 bound of the bf16 kernel's lazy rescaling, so its exact path and the
    rescale of O run on every tile (4-wave schedule at Lk=1000, 8-wave at 8192); 80 also
    drives the probabilities of earlier tiles far below the fp32 range. The fp32 kernel,
    which rescales exactly on every tile, runs the growth of 12 (at 80 its scores reach
    ~600, where fp32 dot products alone err by more than the 1e-4 bar)."""
    B, H, Lq = 1, 2, 300
    alpha = growth / (np.log2(np.e) * np.sqrt(d))          # key scale added per 64 keys
    t = (alpha / 64.0) * np.arange(Lk, dtype=np.float64)
    q = 1.0 + 0.05 * ai.normal_f32((B, H, Lq, d), 61, 0)
    k = (t[None, None, :, None] * (1.0 + 0.01 * ai.normal_f32((B, H, Lk, d), 61, 1))).astype(np.float32)
    v = ai.normal_f32((B, H, Lk, d), 61, 2)
    if dtype == "bf16":
        qs, ks, vs = (ai.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)) for x in (q, k, v))
    else:
        qs, ks, vs = (np.asarray(x, dtype=np.float32) for x in (q, k, v))
    o = lib.attn_fwd(to_dev(qs, dtype), to_dev(ks, dtype), to_dev(vs, dtype), causal=causal)
    import torch
    torch.cuda.synchronize()
    want = oracle.attention(ai.to_f64(qs, dtype), ai.to_f64(ks, dtype), ai.to_f64(vs, dtype),
                            causal=causal)
    assert max_err(from_dev(o), want) <= TOL[dtype]
