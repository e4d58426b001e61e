"""Seeded input generator: determinism, rounding, value distribution."""
import numpy as np
import torch

import attn_inputs as ai


def test_deterministic_and_independent_streams():
    a = ai.make_dense(2, 4, 2, 33, 17, 64, seed=5, kv_len_range=(3, 17))
    b = ai.make_dense(2, 4, 2, 33, 17, 64, seed=5, kv_len_range=(3, 17))
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.kv_len, b.kv_len)):
        assert np.array_equal(x, y)
    assert not np.array_equal(a.k, a.v[..., :a.k.shape[-1]])
    c = ai.make_dense(2, 4, 2, 33, 17, 64, seed=6)
    assert not np.array_equal(a.q, c.q)


def test_bf16_round_to_nearest_even_matches_torch():
    x = ai.normal_f32((1 << 16,), 0, 0) * np.float32(3.0)
    # add exact ties and near-ties
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -130],
                    dtype=np.float32)
    x = np.concatenate([x, ties])
    mine = ai.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    back = ai.bf16_bits_to_f32(mine)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_normal_moments_and_kv_len_range():
    x = ai.normal_f32((1 << 20,), 0, 1).astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.var() - 1.0) < 5e-3
    w = ai.make_dense(8, 1, 1, 1, 4096, 64, seed=0, kv_len_range=(2048, 4096))
    assert w.kv_len.dtype == np.int32 and w.kv_len.min() >= 2048 and w.kv_len.max() <= 4096


def test_bcast_default_map_and_shapes():
    w = ai.make_bcast(64, 2, 8, 8, 16, 32, 128, seed=0)
    assert w.q.shape == (64, 8, 16, 128) and w.k.shape == (2, 8, 32, 128)
    assert np.array_equal(w.cand2user, np.arange(64) // 32)
    assert w.q.dtype == np.uint16


def test_workload_table_shapes():
    spec = ai.WORKLOADS["bcast_Bc1024_Bu32"]
    assert (spec["B_c"], spec["B_u"], spec["Lq"], spec["Lk"], spec["d"]) == (1024, 32, 64, 1024, 128)
    spec = ai.WORKLOADS["gqa_causal_L16384"]
    assert spec["H"] // spec["Hkv"] == 4 and spec["causal"]
    w = ai.make_workload("fp32_tiny")
    assert w.q.dtype == np.float32 and w.q.shape == (1, 1, 128, 64)
