"""The allocation-free entry point attn_fwd_qknorm_noalloc through the C ABI.

It runs the same kernels as attn_fwd_qknorm with the normalised keys in the
library's own device array instead of a caller workspace, so its output must
equal attn_fwd_qknorm's bit for bit. Two calls in a row, the second on a
smaller problem (the array keeps the first call's keys beyond the second's
range), each compared with attn_fwd_qknorm on the same inputs and with the
float64 oracle. The outputs are passed in, so the calls allocate nothing.
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


def _problem(taa, B, H, Hkv, L, d, causal, seed, kv_len_range=None):
    import torch
    w = ai.make_qknorm(B, H, Hkv, L, L, d, causal=causal, seed=seed, kv_len_range=kv_len_range)
    q, k, v = (to_dev(x, "bf16") for x in (w.q, w.k, w.v))
    gq, gk = torch.from_numpy(w.gamma_q).cuda(), torch.from_numpy(w.gamma_k).cuda()
    return w, q, k, v, gq, gk, i32_dev(w.kv_len)


def test_noalloc_matches_workspace_variant_twice(lib):
    import torch
    big = _problem(lib, 1, 8, 4, 700, 128, True, 71)
    small = _problem(lib, 2, 2, 2, 150, 64, False, 72, kv_len_range=(20, 150))
    outs = []
    for w, q, k, v, gq, gk, kvl in (big, small):   # the allocation-free calls, back to back
        o = torch.empty_like(q)
        lib.attn_fwd_qknorm_noalloc(q, k, v, gq, gk, w.eps, o, causal=w.causal, kv_len=kvl)
        outs.append(o)
    torch.cuda.synchronize()
    for (w, q, k, v, gq, gk, kvl), o in zip((big, small), outs):
        ref = lib.attn_fwd_qknorm(q, k, v, gq, gk, w.eps, causal=w.causal, kv_len=kvl)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
        qf, kf, vf = w.f64()
        want = oracle.attention_qknorm(qf, kf, vf, w.gamma_q, w.gamma_k, w.eps, causal=w.causal,
                                       kv_len=w.kv_len)
        assert max_err(from_dev(o), want) <= TOL["bf16"]


def test_noalloc_rejects_a_problem_beyond_its_workspace(lib):
    import torch
    # B * Hkv * Lk * d * 2 = 2 * 8 * 16384 * 128 * 2 bytes = 64 MiB > 32 MiB
    q = torch.zeros((2, 8, 16, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((2, 8, 16384, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.AttnError) as e:
        lib.attn_fwd_qknorm_noalloc(q, k, k)
    assert e.value.status == lib.ATTN_ESCRATCH
