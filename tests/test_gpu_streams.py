"""Work enqueued on a caller's stream that is not torch's current one.

Memory the binding allocates for a call (the output, the uint8 copy of a bool
block mask, the key workspace of the q/k-normalised variant) must belong to
the stream the kernels run on. Otherwise torch's caching allocator can hand a
temporary freed when the call returns to new work on the current stream while
the kernels, still queued behind earlier work on their own stream, have not
read it yet. Each test holds the side stream with a spin kernel, makes the
call, then at once allocates and overwrites memory of the same sizes on the
current stream, and checks the result against the oracle.
"""
import numpy as np
import pytest

import attn_inputs as ai
import oracle
from gpu_util import TOL, from_dev, max_err, to_dev

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 50_000_000   # tens of milliseconds: the call returns long before its kernels run


@pytest.fixture(scope="module")
def lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tiled_attention_attn_amd as taa
    taa.load_library()
    return taa


def _scribble(*sizes):
    """Allocate buffers of the given byte sizes on the current stream and fill them with
    0xFF bytes (a bf16 NaN; a nonzero mask byte) right away."""
    import torch
    return [torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda") for n in sizes for _ in range(2)]


def _held_side_stream():
    import torch
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(SPIN_CYCLES)
    return s


def test_bool_block_mask_on_a_side_stream(lib):
    import torch
    w = ai.make_block_sparse(1, 2, 2, 512, 1024, 128, 128, causal=False, seed=31, density=0.5,
                             mask_heads=2)
    q, k, v = (to_dev(x, "bf16") for x in (w.q, w.k, w.v))
    mask = torch.from_numpy(w.block_mask.astype(bool)).cuda()
    qf, kf, vf = w.f64()
    want = oracle.attention_block_sparse(qf, kf, vf, w.block_mask, w.blk)
    s = _held_side_stream()
    o = lib.attn_fwd_block_sparse(q, k, v, mask, w.blk, stream=s)
    junk = _scribble(mask.numel(), o.numel() * 2)
    s.synchronize()
    torch.cuda.synchronize()
    del junk
    assert max_err(from_dev(o), want) <= TOL["bf16"]


def test_qknorm_workspace_on_a_side_stream(lib):
    import torch
    w = ai.make_qknorm(1, 4, 2, 300, 700, 128, causal=True, seed=32)
    q, k, v = (to_dev(x, "bf16") for x in (w.q, w.k, w.v))
    gq, gk = torch.from_numpy(w.gamma_q).cuda(), torch.from_numpy(w.gamma_k).cuda()
    qf, kf, vf = w.f64()
    want = oracle.attention_qknorm(qf, kf, vf, w.gamma_q, w.gamma_k, w.eps, causal=True)
    s = _held_side_stream()
    o = lib.attn_fwd_qknorm(q, k, v, gq, gk, w.eps, causal=True, stream=s)
    junk = _scribble(k.numel() * 2, o.numel() * 2)
    s.synchronize()
    torch.cuda.synchronize()
    del junk
    assert max_err(from_dev(o), want) <= TOL["bf16"]


def test_linear_outputs_on_a_side_stream(lib):
    import torch
    from test_gpu_ikbo_linear import check
    wl = ai.make_linear(7, 300, 256, 128, 512, shuffle=True, seed=33)
    xu, xc, wt = (to_dev(x, "bf16") for x in (wl.x_user, wl.x_cand, wl.w))
    c2u = torch.from_numpy(wl.cand2user).cuda()
    bias = torch.from_numpy(wl.bias).cuda()
    s = _held_side_stream()
    y, z = lib.ikbo_linear(xu, xc, wt, c2u, bias, stream=s)
    junk = _scribble(z.numel() * 4, y.numel() * 2)
    s.synchronize()
    torch.cuda.synchronize()
    del junk
    check(wl, from_dev(y), from_dev(z))
