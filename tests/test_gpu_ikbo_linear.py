"""The in-kernel broadcast linear layer on the GPU against the float64 oracle,
element by element, through the C ABI.

Error bound, from the arithmetic: products of bf16 values are exact in fp32;
summing K of them in fp32 (in any order, rounding at each addition) errs by at
most (K + 2) * 2^-24 * S per element, with S = sum |x_t w_t| + |bias|; the
bound below doubles that in case the hardware rounds toward zero. A bf16
output adds the final rounding, at most 2^-8 of the value.
"""
import numpy as np
import pytest

import attn_inputs as ai
import oracle
from gpu_util import assert_all_written, from_dev, i32_dev, nan_filled, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tiled_attention_attn_amd as taa
    taa.load_library()
    return taa


def bound(xu, xc, w, c2u, bias, ref, out_dtype):
    """Per-element error bound of the fp32 accumulation (+ bf16 rounding)."""
    K_u = xu.shape[1]
    u = np.clip(c2u, 0, max(xu.shape[0] - 1, 0))
    s = np.abs(xc) @ np.abs(w[:, K_u:]).T
    if K_u:
        s = s + (np.abs(xu) @ np.abs(w[:, :K_u]).T)[u]
    if bias is not None:
        s = s + np.abs(bias)[None, :]
    tol = (w.shape[1] + 2) * 2.0 ** -23 * s
    if out_dtype == "bf16":
        tol = tol + 2.0 ** -8 * np.abs(ref)
    return tol + 1e-30


def run(taa, w, c2u=None):
    import torch
    xu, xc, wt = (to_dev(x, "bf16") for x in (w.x_user, w.x_cand, w.w))
    bias = None if w.bias is None else torch.from_numpy(w.bias).cuda()
    out = torch.bfloat16 if w.out_dtype == "bf16" else torch.float32
    y, z = taa.ikbo_linear(xu, xc, wt, i32_dev(w.cand2user if c2u is None else c2u), bias,
                           out_dtype=out)
    torch.cuda.synchronize()
    return from_dev(y), from_dev(z)


def check(w, y, z, c2u=None):
    c2u = w.cand2user if c2u is None else c2u
    xu, xc, wt, b = w.f64()
    ref = oracle.ikbo_linear(xu, xc, wt, c2u, b)
    ok = ~np.isnan(ref).any(axis=1)
    tol = bound(xu, xc, wt, c2u, b, ref, w.out_dtype)
    err = np.abs(y - ref)
    assert np.all(np.isnan(y[~ok])), "out-of-range users must give NaN rows"
    assert np.all(err[ok] <= tol[ok]), float(np.max(err[ok] / tol[ok]))
    zref = oracle.ikbo_user_partial(xu, wt, b)
    ztol = bound(xu, np.zeros((xu.shape[0], 0)), wt[:, :xu.shape[1]],
                 np.arange(xu.shape[0]), b, zref, "f32")
    assert np.all(np.abs(z - zref) <= ztol)


LINEAR_CASES = [
    # (B_u, B_c, K_u, K_c, N, bias, out dtype, shuffled map)
    (4, 128, 128, 64, 128, True, "bf16", False),     # whole tiles
    (5, 300, 200, 72, 260, True, "bf16", True),      # ragged rows, columns and K tails
    (3, 77, 8, 8, 4, False, "f32", True),            # tiny
    (7, 513, 0, 136, 132, True, "f32", True),        # no user features
    (9, 257, 264, 0, 100, True, "bf16", False),      # no candidate features
    (64, 2048, 1024, 512, 512, True, "bf16", False),
    (33, 1000, 136, 1032, 388, False, "f32", True),
    (6, 0, 64, 64, 128, True, "bf16", False),        # users only: z is still written
    # grids large enough for the bigger tiles (128 x 128, then 256 x 256), ragged
    (16, 2100, 136, 264, 2048, True, "bf16", True),
    (40, 16400, 264, 136, 1028, True, "bf16", True),
]


@pytest.mark.parametrize("case", LINEAR_CASES,
                         ids=lambda c: f"Bu{c[0]}-Bc{c[1]}-Ku{c[2]}-Kc{c[3]}-N{c[4]}-{c[6]}")
def test_ikbo_linear_matches_oracle(lib, case):
    B_u, B_c, K_u, K_c, N, bias, out, shuffle = case
    w = ai.make_linear(B_u, B_c, K_u, K_c, N, bias=bias, out_dtype=out, shuffle=shuffle, seed=41)
    y, z = run(lib, w)
    check(w, y, z)


def test_out_of_range_users_give_nan_rows(lib):
    w = ai.make_linear(4, 200, 64, 64, 128, seed=43)
    c2u = w.cand2user.copy()
    c2u[[0, 7, 199]] = [-1, 4, 1 << 30]
    y, z = run(lib, w, c2u)
    check(w, y, z, c2u)


def test_no_candidate_features_is_the_gathered_user_rows(lib):
    """K_c = 0: y[c] is z[cand2user[c]] rounded to bf16, bit for bit."""
    import torch
    w = ai.make_linear(8, 300, 136, 0, 260, shuffle=True, seed=45)
    y, z = run(lib, w)
    want = torch.from_numpy(z[w.cand2user]).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(y, want)


def test_repeatable(lib):
    w = ai.make_linear(16, 700, 256, 192, 384, shuffle=True, seed=47)
    y1, z1 = run(lib, w)
    y2, z2 = run(lib, w)
    assert np.array_equal(y1, y2) and np.array_equal(z1, z2)


def test_ikbo_linear_full_size_workload_sampled(lib):
    """The full workload, in the launch configuration the bench times; sampled rows
    against the oracle on those candidates."""
    import torch
    w = ai.make_linear_workload("ikbo_linear_Bc65536", seed=0)
    xu, xc, wt = (to_dev(x, "bf16") for x in (w.x_user, w.x_cand, w.w))
    B_u, N = w.x_user.shape[0], w.w.shape[0]
    y = nan_filled(None, (w.x_cand.shape[0], N), torch.bfloat16)
    z = nan_filled(None, (B_u, N), torch.float32)
    lib.ikbo_linear(xu, xc, wt, i32_dev(w.cand2user), torch.from_numpy(w.bias).cuda(), y, z)
    torch.cuda.synchronize()
    assert_all_written(y, "y")
    assert_all_written(z, "z")
    rng = np.random.default_rng(13)
    B_c = w.x_cand.shape[0]
    rows = np.unique(np.concatenate([[0, 127, 128, B_c - 1], rng.integers(0, B_c, 60)]))
    got = y[torch.from_numpy(rows).cuda()].to(torch.float64).cpu().numpy()
    xuf, _, wf, b = w.f64()
    xcf = ai.to_f64(w.x_cand[rows], "bf16")
    ref = oracle.ikbo_linear(xuf, xcf, wf, w.cand2user[rows], b)
    tol = bound(xuf, xcf, wf, w.cand2user[rows], b, ref, "bf16")
    assert np.all(np.abs(got - ref) <= tol)
    users = np.unique(np.concatenate([[0, w.x_user.shape[0] - 1], rng.integers(0, 2048, 8)]))
    zgot = z[torch.from_numpy(users).cuda()].to(torch.float64).cpu().numpy()
    zref = oracle.ikbo_user_partial(xuf[users], wf, b)
    assert np.max(np.abs(zgot - zref)) <= 1e-3


def test_persistent_grid_matches_one_workgroup_per_tile(lib, tmp_path):
    """A grid of one workgroup per slot (several rounds of tiles each) and one
    workgroup per tile (ATTN_GEMM_PERSIST=0, child process) compute every tile
    with the same arithmetic: the outputs are equal bit for bit."""
    import os
    import subprocess
    import sys
    w = ai.make_linear(40, 30000, 264, 136, 1028, shuffle=True, seed=49)   # 118 x 5 tiles of 256
    np.savez(tmp_path / "in.npz", xu=w.x_user, xc=w.x_cand, w=w.w, c2u=w.cand2user, b=w.bias)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = (
        "import sys, numpy as np, torch; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
        "import tiled_attention_attn_amd as taa; from gpu_util import to_dev, from_dev, i32_dev\n"
        "z = np.load(%r)\n"
        "y, zz = taa.ikbo_linear(to_dev(z['xu'], 'bf16'), to_dev(z['xc'], 'bf16'), to_dev(z['w'], 'bf16'),\n"
        "                        i32_dev(z['c2u']), torch.from_numpy(z['b']).cuda())\n"
        "torch.cuda.synchronize(); np.save(%r, from_dev(y))\n"
    )
    outs = {}
    for mode in ("1", "0"):
        out = tmp_path / f"y{mode}.npy"
        env = dict(os.environ, ATTN_GEMM_PERSIST=mode)
        code = script % (root, os.path.join(root, "tests"), str(tmp_path / "in.npz"), str(out))
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                           timeout=300)
        assert r.returncode == 0, r.stderr[-2000:]
        outs[mode] = np.load(out)
    assert np.array_equal(outs["1"], outs["0"], equal_nan=True)


# Forced tile configuration -> (B_c, N) giving more tiles than slots (CUs x workgroups per CU).
PERSIST_CFGS = {
    "0": (16500, 1028),   # 256 x 256 tiles: 65 x 5 = 325 on 256 slots; a 4-column tail
    "1": (8000, 1032),    # 128 x 128: 63 x 9 = 567 on 512 slots; an 8-column last tile
    "2": (8000, 576),     # 128 x 64: 63 x 9 = 567 on 512 slots
    "3": (8000, 576),     # 128 x 64, four stages: 567 on 256 slots
}


@pytest.mark.parametrize("cfg", sorted(PERSIST_CFGS))
def test_persistent_rounds_each_tile_config(lib, tmp_path, cfg):
    """Each tile configuration forced (ATTN_GEMM_CFG, child process) on a grid with more
    tiles than slots: workgroups run several tiles, interior and edge ones, and a tile's bf16
    output is stored behind the next tile's first loads. Candidate depths K_c = 0, 40, 128,
    200 give 0, 1, 2 and 4 stages of K (40 and 200 cut the last one); with an even count the
    last two stages of a tile load the next tile's first two and its row indices. The 2-stage
    case maps some candidates to users out of range (NaN rows, set in the epilogue of tiles
    that start from prefetched operands). Against the oracle."""
    import os
    import subprocess
    import sys
    B_c, N = PERSIST_CFGS[cfg]
    ws = [ai.make_linear(50, B_c, 64, K_c, N, shuffle=True, seed=51 + i)
          for i, K_c in enumerate((0, 40, 128, 200))]
    bad = [3, B_c // 2, B_c - 300, B_c - 1]
    ws[2].cand2user[bad] = [-1, 50, 1 << 30, -7]
    for i, w in enumerate(ws):
        np.savez(tmp_path / f"in{i}.npz", xu=w.x_user, xc=w.x_cand, w=w.w, c2u=w.cand2user,
                 b=w.bias)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = (
        "import sys, numpy as np, torch; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
        "import tiled_attention_attn_amd as taa; from gpu_util import to_dev, from_dev, i32_dev\n"
        "for i in range(%d):\n"
        "    z = np.load('%s/in%%d.npz' %% i)\n"
        "    y, zz = taa.ikbo_linear(to_dev(z['xu'], 'bf16'), to_dev(z['xc'], 'bf16'),\n"
        "                            to_dev(z['w'], 'bf16'), i32_dev(z['c2u']),\n"
        "                            torch.from_numpy(z['b']).cuda())\n"
        "    torch.cuda.synchronize()\n"
        "    np.save('%s/y%%d.npy' %% i, from_dev(y)); np.save('%s/z%%d.npy' %% i, from_dev(zz))\n"
        "    print('case', i, 'done', flush=True)\n"
    ) % (root, os.path.join(root, "tests"), len(ws), tmp_path, tmp_path, tmp_path)
    env = dict(os.environ, ATTN_GEMM_CFG=cfg)
    r = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    for i, w in enumerate(ws):
        check(w, np.load(tmp_path / f"y{i}.npy"), np.load(tmp_path / f"z{i}.npy"))


def test_four_stage_ring_remainders(lib, tmp_path):
    """Configuration 3 (four LDS stages, loads three stages ahead) forced on K depths whose
    stage counts leave every remainder of the ring: 3, 5, 6 and 7 stages of 64 (some cut by
    K), in the fp32 user half (K_u) and the bf16 candidate half (K_c). Against the oracle."""
    import os
    import subprocess
    import sys
    shapes = [(136, 320), (384, 448), (200, 392), (448, 136)]   # (K_u, K_c)
    ws = [ai.make_linear(40, 1500, K_u, K_c, 264, shuffle=True, seed=61 + i)
          for i, (K_u, K_c) in enumerate(shapes)]
    for i, w in enumerate(ws):
        np.savez(tmp_path / f"in{i}.npz", xu=w.x_user, xc=w.x_cand, w=w.w, c2u=w.cand2user,
                 b=w.bias)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = (
        "import sys, numpy as np, torch; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
        "import tiled_attention_attn_amd as taa; from gpu_util import to_dev, from_dev, i32_dev\n"
        "for i in range(%d):\n"
        "    z = np.load('%s/in%%d.npz' %% i)\n"
        "    y, zz = taa.ikbo_linear(to_dev(z['xu'], 'bf16'), to_dev(z['xc'], 'bf16'),\n"
        "                            to_dev(z['w'], 'bf16'), i32_dev(z['c2u']),\n"
        "                            torch.from_numpy(z['b']).cuda())\n"
        "    torch.cuda.synchronize()\n"
        "    np.save('%s/y%%d.npy' %% i, from_dev(y)); np.save('%s/z%%d.npy' %% i, from_dev(zz))\n"
        "    print('case', i, 'done', flush=True)\n"
    ) % (root, os.path.join(root, "tests"), len(ws), tmp_path, tmp_path, tmp_path)
    env = dict(os.environ, ATTN_GEMM_CFG="3")
    r = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    for i, w in enumerate(ws):
        check(w, np.load(tmp_path / f"y{i}.npy"), np.load(tmp_path / f"z{i}.npy"))
