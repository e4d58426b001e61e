"""Keys past the valid ones are never read: NaN in the K/V rows past kv_len (padding a
caller may leave uninitialised) or in the memory right after the last row must not
reach the output. Masked keys get probability 0, and 0 * NaN would poison the row if
those V rows were read; the kernels' loads end with the last valid row.
"""
import numpy as np
import pytest

import attn_inputs as ai
import oracle
from gpu_util import TOL, from_dev, i32_dev, max_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tiled_attention_attn_amd as taa
    taa.load_library()
    return taa


def _poison_past_kv_len(x, kv_len):
    """x: [B, Hkv, Lk, d] host array of bf16 bits or float32; NaN in rows >= kv_len[b]."""
    x = x.copy()
    nan = np.uint16(0x7FC0) if x.dtype == np.uint16 else np.float32("nan")
    for b, n in enumerate(kv_len):
        x[b, :, n:, :] = nan
    return x


def _in_nan_tail(x, dtype):
    """A device tensor holding x, placed at the end of a larger allocation whose tail
    (right after x) is NaN."""
    import torch
    t = to_dev(x, dtype)
    n = t.numel()
    buf = torch.full((n + 4096,), float("nan"), dtype=t.dtype, device="cuda")
    buf[:n] = t.reshape(-1)
    return buf[:n].view(t.shape)


CASES = [
    # (B, H, Hkv, Lq, Lk, d, dtype, causal)
    (3, 4, 2, 100, 300, 128, "bf16", False),    # 4-wave schedule
    (3, 2, 2, 130, 260, 64, "bf16", True),      # 4-wave, d = 64
    (2, 2, 1, 300, 4500, 128, "bf16", False),   # 8-wave schedule
    (2, 2, 2, 70, 150, 64, "f32", False),       # fp32 path
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_nan_past_kv_len_and_after_the_last_row(lib, case):
    import torch
    B, H, Hkv, Lq, Lk, d, dtype, causal = case
    w = ai.make_dense(B, H, Hkv, Lq, Lk, d, dtype=dtype, causal=causal, seed=91,
                      kv_len_range=(1, Lk - 1))
    k = _poison_past_kv_len(w.k, w.kv_len)
    v = _poison_past_kv_len(w.v, w.kv_len)
    q = to_dev(w.q, dtype)
    kd, vd = _in_nan_tail(k, dtype), _in_nan_tail(v, dtype)
    o = lib.attn_fwd(q, kd, vd, causal=causal, kv_len=i32_dev(w.kv_len))
    torch.cuda.synchronize()
    got = from_dev(o)
    qf, kf, vf = w.f64()      # the unpoisoned values: rows past kv_len do not matter
    ref = oracle.attention(qf, kf, vf, causal=causal, kv_len=w.kv_len)
    assert not np.isnan(got).any(), "padding past kv_len reached the output"
    assert max_err(got, ref) <= TOL[dtype]


def test_nan_past_user_kv_len_in_the_broadcast_variant(lib):
    import torch
    B_c, B_u, Lk = 24, 3, 200
    w = ai.make_bcast(B_c, B_u, 2, 2, 64, Lk, 128, seed=92, shuffle=True, kv_len_range=(1, Lk - 1))
    k = _poison_past_kv_len(w.k, w.kv_len)
    v = _poison_past_kv_len(w.v, w.kv_len)
    q = to_dev(w.q, "bf16")
    o = lib.attn_fwd_bcast(q, _in_nan_tail(k, "bf16"), _in_nan_tail(v, "bf16"),
                           i32_dev(w.cand2user), kv_len=i32_dev(w.kv_len))
    torch.cuda.synchronize()
    got = from_dev(o)
    qf, kf, vf = w.f64()
    ref = oracle.attention_bcast(qf, kf, vf, w.cand2user, kv_len=w.kv_len)
    assert not np.isnan(got).any()
    assert max_err(got, ref) <= TOL["bf16"]


@pytest.mark.parametrize("L", [2000, 4200])   # 4-wave and 8-wave schedules
def test_inf_in_v_stays_out_of_tiles_that_do_not_hold_it(lib, L):
    """Causal: V row 100 (key tile 1) holds +Inf. Rows 0..63 need key tile 0 only, so they
    must stay finite and match the oracle: no product of theirs may multiply that row, not
    even by a zero probability (0 * Inf = NaN), including the 8-wave schedule's first, empty
    PV product. (Rows 64..99 share the tile with key 100 and are masked against it; their
    zero probabilities still multiply it, as the header documents.)"""
    import torch
    B, H, Hkv, d = 1, 2, 2, 128
    w = ai.make_dense(B, H, Hkv, L, L, d, causal=True, seed=93)
    v = w.v.copy()
    v[:, :, 100, :] = np.uint16(0x7F80)     # bf16 +Inf
    q, k = to_dev(w.q, "bf16"), to_dev(w.k, "bf16")
    o = lib.attn_fwd(q, k, to_dev(v, "bf16"), causal=True)
    torch.cuda.synchronize()
    got = from_dev(o)[:, :, :64]
    assert np.isfinite(got).all(), "a row whose tiles do not hold the Inf key went non-finite"
    qf, kf, vf = w.f64()
    rows = np.arange(64)
    for h in range(H):
        ref = oracle.attention_rows(qf, kf, vf, 0, h, rows, causal=True)
        assert max_err(got[0, h], ref) <= TOL["bf16"]
