"""Fixed-block sparse attention on the GPU against the float64 oracle,
element by element, through the C ABI."""
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


def run_sparse(taa, w, mask=None):
    import torch
    q, k, v = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v))
    bm = torch.from_numpy(np.ascontiguousarray(w.block_mask if mask is None else mask)).cuda()
    o = taa.attn_fwd_block_sparse(q, k, v, bm, w.blk, causal=w.causal, kv_len=i32_dev(w.kv_len),
                                  scale=w.scale or 0.0)
    torch.cuda.synchronize()
    return from_dev(o)


def ref_sparse(w, mask=None):
    q, k, v = w.f64()
    return oracle.attention_block_sparse(q, k, v, w.block_mask if mask is None else mask, w.blk,
                                         causal=w.causal, kv_len=w.kv_len, scale=w.scale)


SPARSE_CASES = [
    # (B, H, Hkv, Lq, Lk, d, dtype, causal, blk, mask_heads, density or None (pattern), kv_len)
    (1, 2, 2, 512, 512, 128, "bf16", False, 128, 1, 0.5, None),
    (2, 4, 2, 600, 700, 128, "bf16", True, 128, 4, 0.6, None),       # ragged edges, per-head
    (1, 2, 1, 777, 1000, 64, "bf16", False, 256, 2, 0.4, (300, 1000)),
    (1, 2, 2, 640, 640, 128, "bf16", True, 128, 1, None, None),      # local band + global
    (1, 2, 2, 4500, 4600, 128, "bf16", True, 256, 2, 0.3, None),     # 8-wave schedule
    (1, 2, 2, 4200, 4200, 128, "bf16", False, 384, 1, 0.5, None),    # blk not a power of two
    (1, 2, 2, 300, 300, 64, "f32", True, 128, 2, 0.6, None),
    (1, 1, 1, 256, 512, 128, "f32", False, 256, 1, 0.5, None),
]


def _random_sparse_cases(n=5, seed=2029):
    """Seeded block-sparse problems: block sizes of 128-512, random masks per head or
    shared, ragged edges, both head dims, with or without kv_len."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        Hkv = int(rng.integers(1, 3))
        H = Hkv * int(rng.choice([1, 2]))
        blk = 128 * int(rng.integers(1, 5))
        Lq, Lk = int(rng.integers(1, 1500)), int(rng.integers(1, 1500))
        kvr = (int(rng.integers(0, Lk)), Lk) if rng.random() < 0.4 else None
        cases.append((int(rng.integers(1, 3)), H, Hkv, Lq, Lk, int(rng.choice([64, 128])), "bf16",
                      bool(rng.random() < 0.5), blk, int(rng.choice([1, H])),
                      float(rng.uniform(0.2, 0.8)), kvr))
    return cases


SPARSE_CASES += _random_sparse_cases()


@pytest.mark.parametrize("case", SPARSE_CASES,
                         ids=lambda c: f"{c[6]}-d{c[5]}-c{int(c[7])}-L{c[3]}x{c[4]}-blk{c[8]}")
def test_block_sparse_matches_oracle(lib, case):
    B, H, Hkv, Lq, Lk, d, dtype, causal, blk, mh, dens, kvr = case
    if dens is None:
        w = ai.make_block_sparse(B, H, Hkv, Lq, Lk, d, blk, dtype=dtype, causal=causal, seed=31,
                                 window=2, n_global=1, mask_heads=mh, kv_len_range=kvr)
    else:
        w = ai.make_block_sparse(B, H, Hkv, Lq, Lk, d, blk, dtype=dtype, causal=causal, seed=31,
                                 density=dens, mask_heads=mh, kv_len_range=kvr)
    got = run_sparse(lib, w)
    assert max_err(got, ref_sparse(w)) <= TOL[dtype]


def test_empty_query_blocks_give_zero_rows(lib):
    w = ai.make_block_sparse(1, 2, 2, 384, 384, 128, 128, seed=33, density=1.0, mask_heads=2)
    w.block_mask[0, 1, :] = 0          # head 0, rows 128..255: no key block at all
    w.block_mask[1, :, :] = 0          # head 1: nothing
    got = run_sparse(lib, w)
    assert np.all(got[0, 0, 128:256] == 0) and np.all(got[0, 1] == 0)
    assert max_err(got, ref_sparse(w)) <= TOL["bf16"]


@pytest.mark.parametrize("Lk,blk", [(1000, 128), (4400, 256)])
def test_all_ones_mask_equals_dense_kernel(lib, Lk, blk):
    """Every block set: the same tiles in the same order as the dense kernel, bit for bit."""
    import torch
    w = ai.make_block_sparse(1, 2, 2, 600, Lk, 128, blk, causal=True, seed=35, density=1.0)
    got = run_sparse(lib, w)
    q, k, v = (to_dev(x, "bf16") for x in (w.q, w.k, w.v))
    o = lib.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert np.array_equal(got, from_dev(o))


def test_block_sparse_full_size_workload_sampled(lib):
    import torch
    w = ai.make_workload("block_sparse_L16384", seed=0)
    q, k, v = (to_dev(x, w.dtype) for x in (w.q, w.k, w.v))
    o = nan_filled(q)
    lib.attn_fwd_block_sparse(q, k, v, torch.from_numpy(w.block_mask).cuda(), w.blk, o,
                              causal=w.causal)
    torch.cuda.synchronize()
    assert_all_written(o)
    rng = np.random.default_rng(11)
    B, H, Lq, _ = w.q.shape
    worst = 0.0
    for b, h in [(0, 0), (0, H - 1)] + [(0, int(rng.integers(H))) for _ in range(3)]:
        rows = np.unique(np.concatenate([[0, 255, 256, 2047, 2048, Lq - 1],
                                         rng.integers(0, Lq, 8)]))
        got = o[b, h, torch.from_numpy(rows).cuda()].to(torch.float64).cpu().numpy()
        qf, kf, vf = (ai.to_f64(x, w.dtype) for x in
                      (w.q[b:b + 1, h:h + 1], w.k[b:b + 1, h:h + 1], w.v[b:b + 1, h:h + 1]))
        ref = oracle.attention_block_sparse_rows(qf, kf, vf, w.block_mask, w.blk, 0, 0, rows,
                                                 causal=w.causal)
        worst = max(worst, max_err(got, ref))
    assert worst <= TOL[w.dtype], worst


@pytest.mark.parametrize("Lk,causal", [(1000, False), (4400, True)], ids=lambda v: str(v))
def test_reference_moves_across_skipped_blocks(lib, Lk, causal):
    """Scores grow by about 12 (base 2, after the softmax scale) per 64 keys, and about half
    of the key blocks are skipped: the running maximum jumps past the lazy-rescale bound on
    every kept tile, often right after a skipped block (4-wave schedule at Lk=1000, 8-wave at
    4400)."""
    import torch
    B, H, Lq, d, blk = 1, 2, 600, 128, 128
    alpha = 12.0 / (np.log2(np.e) * np.sqrt(d))
    t = (alpha / 64.0) * np.arange(Lk, dtype=np.float64)
    q = 1.0 + 0.05 * ai.normal_f32((B, H, Lq, d), 63, 0)
    k = t[None, None, :, None] * (1.0 + 0.01 * ai.normal_f32((B, H, Lk, d), 63, 1))
    v = ai.normal_f32((B, H, Lk, d), 63, 2)
    qb, kb, vb = (ai.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)) for x in (q, k, v))
    nq, nk = -(-Lq // blk), -(-Lk // blk)
    mask = (np.random.default_rng(63).random((H, nq, nk)) < 0.5).astype(np.uint8)
    mask[:, :, 0] = 1                                   # every row keeps at least one block
    o = lib.attn_fwd_block_sparse(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"),
                                  torch.from_numpy(mask).cuda(), blk, causal=causal)
    torch.cuda.synchronize()
    want = oracle.attention_block_sparse(ai.to_f64(qb, "bf16"), ai.to_f64(kb, "bf16"),
                                         ai.to_f64(vb, "bf16"), mask, blk, causal=causal)
    assert max_err(from_dev(o), want) <= TOL["bf16"]
