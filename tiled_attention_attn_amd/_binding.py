"""ctypes binding of libattn.so with the same entry-point names as include/attn.h.

Argument marshalling only: shapes, dtypes and devices of torch tensors are
checked and their device pointers handed to the C ABI. Every step of the
computation runs in the library's HIP kernels; there is no fallback path.

Streams: every call takes `stream=` (a torch stream; default torch's current
one) and enqueues its kernels there without synchronising. Tensors the binding
allocates for a call (outputs not passed in, the uint8 copy of a bool block
mask, the key workspace) are allocated with that stream current, so torch's
caching allocator reuses them only in that stream's order.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_ELAUNCH, ATTN_ESCRATCH = 0, -1, -2, -3, -4
ATTN_F32, ATTN_BF16 = 0, 1

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"attention library error {status}: {msg}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libattn.so (once). Raises RuntimeError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m tiled_attention_attn_amd.build` "
            "(hipcc, gfx950). There is no fallback implementation.")
    # torch ships its own HIP runtime under the same soname as the system one
    # this library links; whichever loads first serves the process. Loading
    # torch first keeps torch on its own runtime and this library on the same
    # one (loaded the other way round, kernel launches failed).
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, f32, i32, vp]
    lib.attn_fwd.restype = i32
    lib.attn_fwd_bcast.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                   vp, f32, i32, vp]
    lib.attn_fwd_bcast.restype = i32
    lib.attn_fwd_bcast_grouped.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                           i32, i32, vp, f32, i32, vp]
    lib.attn_fwd_bcast_grouped.restype = i32
    lib.attn_bcast_group.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.attn_bcast_group.restype = i32
    lib.attn_fwd_jagged.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    f32, i32, vp]
    lib.attn_fwd_jagged.restype = i32
    lib.attn_fwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                          i32, i32, vp, f32, i32, vp]
    lib.attn_fwd_block_sparse.restype = i32
    lib.attn_fwd_qknorm.argtypes = [vp, vp, vp, vp, vp, vp, f32, vp, i32, i32, i32, i32, i32,
                                    i32, i32, vp, f32, i32, vp]
    lib.attn_fwd_qknorm.restype = i32
    lib.attn_fwd_qknorm_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32,
                                            i32, i32, i32, vp, f32, i32, vp]
    lib.attn_fwd_qknorm_noalloc.restype = i32
    lib.ikbo_linear.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.ikbo_linear.restype = i32
    lib.attn_strerror.argtypes = [i32]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = i32
    i64 = ctypes.c_int64
    lib.attn_ceiling_mfma_bf16.argtypes = [vp, i64, vp, i32, i32, i32, vp]
    lib.attn_ceiling_mfma16_bf16.argtypes = [vp, i64, vp, i32, i32, i32, vp]
    lib.attn_ceiling_exp2.argtypes = [vp, i32, i32, vp]
    lib.attn_ceiling_fma.argtypes = [vp, i32, i32, vp]
    lib.attn_ceiling_exp2_fma.argtypes = [vp, i32, i32, vp]
    lib.attn_ceiling_lds_read.argtypes = [vp, i32, i32, i32, vp]
    lib.attn_ceiling_copy.argtypes = [vp, vp, i64, vp]
    for fn in (lib.attn_ceiling_mfma_bf16, lib.attn_ceiling_mfma16_bf16, lib.attn_ceiling_exp2,
               lib.attn_ceiling_fma,
               lib.attn_ceiling_exp2_fma,
               lib.attn_ceiling_lds_read, lib.attn_ceiling_copy):
        fn.restype = i32
    _lib = lib
    return lib


def attn_strerror(status: int) -> str:
    return load_library().attn_strerror(int(status)).decode()


def attn_version() -> int:
    return int(load_library().attn_version())


def _check(status: int):
    if status != ATTN_OK:
        raise AttnError(status, attn_strerror(status))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _prep(q, k, v, o, extra, stream=None):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [batch, heads, seq, d]")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [batch, heads, seq, d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if q.shape[3] != k.shape[3]:
        raise ValueError("q and k must have the same head dimension")
    if o is None:
        o = _on(stream, lambda: torch.empty_like(q))
    elif o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous() or not o.is_cuda:
        raise ValueError("o must be a contiguous device tensor shaped and typed like q")
    for name, t in extra.items():
        if t is not None and (t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    return o


def _torch_stream(stream):
    """The torch stream the work is enqueued on: `stream`, or torch's current one."""
    import torch
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream):
    return ctypes.c_void_p(_torch_stream(stream).cuda_stream)


def _on(stream, fn):
    """Run fn (an allocation, or a conversion that allocates) with `stream` current, so that
    torch's caching allocator ties the new memory to the stream the kernels use: memory
    freed by the caller (or, for temporaries, when this call returns) is then only reused
    by work ordered after those kernels on that stream."""
    import torch
    with torch.cuda.stream(_torch_stream(stream)):
        return fn()


def attn_fwd(q, k, v, o=None, *, causal=False, kv_len=None, scale=0.0, stream=None):
    """O = softmax(scale * Q K^T + mask) V on the GPU; returns o.

    q [B,H,Lq,d], k/v [B,Hkv,Lk,d] (bf16 or fp32, contiguous, on the device);
    kv_len: int32 [B] device tensor or None; scale 0 means 1/sqrt(d).
    Enqueued on `stream` (default: torch's current stream); not synchronised.
    """
    lib = load_library()
    o = _prep(q, k, v, o, {"kv_len": kv_len}, stream)
    B, H, Lq, d = q.shape
    if k.shape[0] != B:
        raise ValueError("k/v batch must equal q batch (use attn_fwd_bcast for a broadcast)")
    if kv_len is not None and kv_len.numel() != B:
        raise ValueError("kv_len must have one entry per batch element")
    _check(lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, k.shape[1], Lq, k.shape[2], d,
                        int(bool(causal)), _ptr(kv_len), float(scale), _dtype_code(q),
                        _stream(stream)))
    return o


def attn_fwd_bcast(q, k, v, cand2user, o=None, *, causal=False, kv_len=None, scale=0.0,
                   order=None, stream=None):
    """In-kernel broadcast attention: candidate c uses user cand2user[c]'s K/V.

    q [B_c,H,Lq,d], k/v [B_u,Hkv,Lk,d], cand2user int32 [B_c] device tensor,
    kv_len int32 [B_u] device tensor or None. Returns o [B_c,H,Lq,d].
    order: optional int32 [B_c] device tensor, the order in which candidates are packed
    into workgroups (a permutation, e.g. from bcast_group); calls attn_fwd_bcast_grouped.
    """
    lib = load_library()
    o = _prep(q, k, v, o, {"cand2user": cand2user, "kv_len": kv_len, "order": order}, stream)
    B_c, H, Lq, d = q.shape
    B_u = k.shape[0]
    if cand2user.numel() != B_c:
        raise ValueError("cand2user must have one entry per candidate")
    if kv_len is not None and kv_len.numel() != B_u:
        raise ValueError("kv_len must have one entry per user")
    if order is None:
        _check(lib.attn_fwd_bcast(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(cand2user), B_c, B_u,
                                  H, k.shape[1], Lq, k.shape[2], d, int(bool(causal)),
                                  _ptr(kv_len), float(scale), _dtype_code(q), _stream(stream)))
        return o
    if order.numel() != B_c:
        raise ValueError("order must have one entry per candidate")
    _check(lib.attn_fwd_bcast_grouped(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(cand2user),
                                      _ptr(order), B_c, B_u, H, k.shape[1], Lq, k.shape[2], d,
                                      int(bool(causal)), _ptr(kv_len), float(scale),
                                      _dtype_code(q), _stream(stream)))
    return o


def bcast_group(cand2user, B_u, order=None, *, work=None, stream=None):
    """A permutation of the candidates that keeps each user's candidates together (users
    in increasing order, out-of-range users last), computed on the device
    (attn_bcast_group). Returns order, an int32 [B_c] device tensor. work: optional
    int32 device tensor of at least B_u + 1 entries (allocated here if None)."""
    import torch
    lib = load_library()
    if cand2user.dtype != torch.int32 or not cand2user.is_cuda or not cand2user.is_contiguous():
        raise ValueError("cand2user must be a contiguous int32 device tensor")
    B_c = cand2user.numel()
    if order is None:
        order = _on(stream, lambda: torch.empty(B_c, dtype=torch.int32, device=cand2user.device))
    elif order.numel() != B_c or order.dtype != torch.int32 or not order.is_contiguous():
        raise ValueError("order must be a contiguous int32 device tensor with B_c entries")
    if work is None:
        work = _on(stream, lambda: torch.empty(int(B_u) + 1, dtype=torch.int32,
                                               device=cand2user.device))
    elif (work.numel() < int(B_u) + 1 or work.dtype != torch.int32 or not work.is_cuda
          or not work.is_contiguous()):
        raise ValueError("work must be a contiguous int32 device tensor of B_u + 1 entries")
    _check(lib.attn_bcast_group(_ptr(cand2user), B_c, int(B_u), _ptr(order), _ptr(work),
                                _stream(stream)))
    return order


def attn_fwd_jagged(q, k, v, q_offsets, kv_offsets, max_lq, max_lk, o=None, *, causal=False,
                    scale=0.0, stream=None):
    """Jagged attention: sequence b's queries q[q_offsets[b]:q_offsets[b+1]] attend over
    k/v[kv_offsets[b]:kv_offsets[b+1]] only.

    q [total_q,H,d], k/v [total_kv,Hkv,d] (bf16 or fp32, contiguous, on the device);
    q_offsets / kv_offsets: int32 [B+1] device tensors; max_lq / max_lk: host ints
    bounding the sequence lengths. Returns o [total_q,H,d].
    """
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-D device tensor [tokens, heads, d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if k.shape != v.shape or q.shape[2] != k.shape[2]:
        raise ValueError("k and v must match, and share d with q")
    for name, t in (("q_offsets", q_offsets), ("kv_offsets", kv_offsets)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous() or t.dim() != 1:
            raise ValueError(f"{name} must be a contiguous 1-D int32 device tensor")
    if q_offsets.numel() != kv_offsets.numel() or q_offsets.numel() < 1:
        raise ValueError("q_offsets and kv_offsets must both hold B+1 entries")
    if o is None:
        o = _on(stream, lambda: torch.empty_like(q))
    elif o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous() or not o.is_cuda:
        raise ValueError("o must be a contiguous device tensor shaped and typed like q")
    B = q_offsets.numel() - 1
    _, H, d = q.shape
    _check(lib.attn_fwd_jagged(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(q_offsets),
                               _ptr(kv_offsets), B, H, k.shape[1], int(max_lq), int(max_lk), d,
                               int(bool(causal)), float(scale), _dtype_code(q), _stream(stream)))
    return o


def attn_fwd_block_sparse(q, k, v, block_mask, blk, o=None, *, causal=False, kv_len=None,
                          scale=0.0, stream=None):
    """Fixed-block sparse attention: query block qb attends to key block kb only where
    block_mask[h or 0, qb, kb] is nonzero.

    q [B,H,Lq,d], k/v [B,Hkv,Lk,d] as attn_fwd; block_mask: uint8 (or bool) device tensor
    [1 or H, ceil(Lq/blk), ceil(Lk/blk)]; blk a multiple of 128. Returns o.
    """
    import torch
    lib = load_library()
    o = _prep(q, k, v, o, {"kv_len": kv_len}, stream)
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if k.shape[0] != B:
        raise ValueError("k/v batch must equal q batch")
    if block_mask.dtype == torch.bool:   # converted on the kernels' stream, ahead of them
        block_mask = _on(stream, lambda: block_mask.to(torch.uint8))
    if (block_mask.dtype != torch.uint8 or not block_mask.is_cuda or not block_mask.is_contiguous()
            or block_mask.dim() != 3):
        raise ValueError("block_mask must be a contiguous 3-D uint8 device tensor")
    nqb, nkb = -(-Lq // blk), -(-Lk // blk)
    if block_mask.shape[0] not in (1, H) or tuple(block_mask.shape[1:]) != (nqb, nkb):
        raise ValueError(f"block_mask must be [1 or {H}, {nqb}, {nkb}] for blk={blk}")
    if kv_len is not None and kv_len.numel() != B:
        raise ValueError("kv_len must have one entry per batch element")
    _check(lib.attn_fwd_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(block_mask),
                                     block_mask.shape[0], int(blk), B, H, k.shape[1], Lq, Lk, d,
                                     int(bool(causal)), _ptr(kv_len), float(scale),
                                     _dtype_code(q), _stream(stream)))
    return o


def attn_fwd_qknorm(q, k, v, gamma_q=None, gamma_k=None, eps=1e-6, o=None, k_norm=None, *,
                    causal=False, kv_len=None, scale=0.0, stream=None):
    """Attention on RMS-normalised queries and keys; returns o.

    q [B,H,Lq,d], k/v [B,Hkv,Lk,d] bf16 as attn_fwd; gamma_q / gamma_k float32 [d] device
    tensors or None (ones); k_norm: bf16 workspace shaped like k (allocated when None),
    written with the normalised keys.
    """
    import torch
    lib = load_library()
    o = _prep(q, k, v, o, {"kv_len": kv_len}, stream)
    B, H, Lq, d = q.shape
    if k.shape[0] != B:
        raise ValueError("k/v batch must equal q batch")
    if kv_len is not None and kv_len.numel() != B:
        raise ValueError("kv_len must have one entry per batch element")
    for name, g in (("gamma_q", gamma_q), ("gamma_k", gamma_k)):
        if g is not None and (g.dtype != torch.float32 or not g.is_cuda or not g.is_contiguous()
                              or g.numel() != d):
            raise ValueError(f"{name} must be a contiguous float32 device tensor with d entries")
    if k_norm is None:
        k_norm = _on(stream, lambda: torch.empty_like(k))
    elif (k_norm.shape != k.shape or k_norm.dtype != k.dtype or not k_norm.is_cuda
          or not k_norm.is_contiguous()):
        raise ValueError("k_norm must be a contiguous device tensor shaped and typed like k")
    _check(lib.attn_fwd_qknorm(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(gamma_q), _ptr(gamma_k),
                               float(eps), _ptr(k_norm), B, H, k.shape[1], Lq, k.shape[2], d,
                               int(bool(causal)), _ptr(kv_len), float(scale), _dtype_code(q),
                               _stream(stream)))
    return o


def attn_fwd_qknorm_noalloc(q, k, v, gamma_q=None, gamma_k=None, eps=1e-6, o=None, *,
                            causal=False, kv_len=None, scale=0.0, stream=None):
    """attn_fwd_qknorm with the normalised keys in the library's own device workspace
    (32 MiB per GPU; no device memory is allocated by the library). Calls whose work
    overlaps on one GPU share that workspace and must be serialised. Returns o (allocated
    on `stream` when None: pass o for a call that allocates nothing at all)."""
    import torch
    lib = load_library()
    o = _prep(q, k, v, o, {"kv_len": kv_len}, stream)
    B, H, Lq, d = q.shape
    if k.shape[0] != B:
        raise ValueError("k/v batch must equal q batch")
    if kv_len is not None and kv_len.numel() != B:
        raise ValueError("kv_len must have one entry per batch element")
    for name, g in (("gamma_q", gamma_q), ("gamma_k", gamma_k)):
        if g is not None and (g.dtype != torch.float32 or not g.is_cuda or not g.is_contiguous()
                              or g.numel() != d):
            raise ValueError(f"{name} must be a contiguous float32 device tensor with d entries")
    _check(lib.attn_fwd_qknorm_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(gamma_q),
                                       _ptr(gamma_k), float(eps), B, H, k.shape[1], Lq,
                                       k.shape[2], d, int(bool(causal)), _ptr(kv_len),
                                       float(scale), _dtype_code(q), _stream(stream)))
    return o


def ikbo_linear(x_user, x_cand, w, cand2user, bias=None, y=None, z=None, *, out_dtype=None,
                stream=None):
    """In-kernel broadcast linear layer; returns (y, z).

    y[c] = concat(x_user[cand2user[c]], x_cand[c]) @ w.T + bias, computed as
    x_cand @ w[:, K_u:].T plus row cand2user[c] of z = x_user @ w[:, :K_u].T + bias.
    x_user [B_u,K_u], x_cand [B_c,K_c], w [N,K_u+K_c]: contiguous bf16 device tensors;
    cand2user int32 [B_c]; bias fp32 [N] or None; y [B_c,N] bf16 (default) or fp32;
    z fp32 [B_u,N] (allocated when None).
    """
    import torch
    lib = load_library()
    for name, t in (("x_user", x_user), ("x_cand", x_cand), ("w", w)):
        if (not t.is_cuda or not t.is_contiguous() or t.dim() != 2
                or t.dtype != torch.bfloat16):
            raise ValueError(f"{name} must be a contiguous 2-D bfloat16 device tensor")
    B_u, K_u = x_user.shape
    B_c, K_c = x_cand.shape
    N = w.shape[0]
    if w.shape[1] != K_u + K_c:
        raise ValueError(f"w must be [N, {K_u + K_c}] (user columns, then candidate columns)")
    if (cand2user.dtype != torch.int32 or not cand2user.is_cuda or not cand2user.is_contiguous()
            or cand2user.numel() != B_c):
        raise ValueError("cand2user must be a contiguous int32 device tensor with B_c entries")
    if bias is not None and (bias.dtype != torch.float32 or not bias.is_cuda
                             or not bias.is_contiguous() or bias.numel() != N):
        raise ValueError("bias must be a contiguous float32 device tensor with N entries")
    if y is None:
        y = _on(stream, lambda: torch.empty((B_c, N), dtype=out_dtype or torch.bfloat16,
                                            device=x_cand.device))
    elif (tuple(y.shape) != (B_c, N) or not y.is_cuda or not y.is_contiguous()
          or y.dtype not in (torch.bfloat16, torch.float32)):
        raise ValueError("y must be a contiguous [B_c, N] bfloat16 or float32 device tensor")
    if z is None:
        z = _on(stream, lambda: torch.empty((B_u, N), dtype=torch.float32, device=x_user.device))
    elif (tuple(z.shape) != (B_u, N) or z.dtype != torch.float32 or not z.is_cuda
          or not z.is_contiguous()):
        raise ValueError("z must be a contiguous [B_u, N] float32 device tensor")
    _check(lib.ikbo_linear(_ptr(x_user), _ptr(x_cand), _ptr(w), _ptr(bias), _ptr(cand2user),
                           _ptr(y), _ptr(z), B_u, B_c, K_u, K_c, N, _dtype_code(y),
                           _stream(stream)))
    return y, z


# --- ceiling microbenchmarks (include/attn_ceiling.h) ----------------------------------------

def _probe_check(status: int, name: str):
    if status != 0:
        raise RuntimeError(f"{name}: status {status}")


def ceiling_mfma_bf16(operands, out, workgroups, waves, iters, stream=None):
    """Enqueue the bf16 matrix-core probe. operands: bf16 device tensor holding
    operand_lanes x 128 values (16 operand vectors of 8 per lane); out: float32 device
    tensor of workgroups*waves*64 entries. FLOPs = workgroups*waves*iters*8*32768."""
    lanes = operands.numel() // 128
    if out.numel() < workgroups * waves * 64 or lanes < 1:
        raise ValueError("ceiling_mfma_bf16: buffers too small")
    _probe_check(load_library().attn_ceiling_mfma_bf16(_ptr(operands), lanes, _ptr(out),
                                                       int(workgroups), int(waves), int(iters),
                                                       _stream(stream)), "attn_ceiling_mfma_bf16")


def ceiling_mfma16_bf16(operands, out, workgroups, waves, iters, stream=None):
    """Enqueue the same probe on v_mfma_f32_16x16x32_bf16 (the same arguments).
    FLOPs = workgroups*waves*iters*16*16384."""
    lanes = operands.numel() // 128
    if out.numel() < workgroups * waves * 64 or lanes < 1:
        raise ValueError("ceiling_mfma16_bf16: buffers too small")
    _probe_check(load_library().attn_ceiling_mfma16_bf16(_ptr(operands), lanes, _ptr(out),
                                                         int(workgroups), int(waves), int(iters),
                                                         _stream(stream)), "attn_ceiling_mfma16_bf16")


def ceiling_exp2(out, workgroups, iters, stream=None):
    """Enqueue the v_exp_f32 probe: workgroups*256*iters*16 exponentials."""
    if out.numel() < workgroups * 256:
        raise ValueError("ceiling_exp2: out too small")
    _probe_check(load_library().attn_ceiling_exp2(_ptr(out), int(workgroups), int(iters),
                                                  _stream(stream)), "attn_ceiling_exp2")


def ceiling_fma(out, workgroups, iters, stream=None):
    """Enqueue the scalar fp32 FMA probe: workgroups*256*iters*16 FMAs."""
    if out.numel() < workgroups * 256:
        raise ValueError("ceiling_fma: out too small")
    _probe_check(load_library().attn_ceiling_fma(_ptr(out), int(workgroups), int(iters),
                                                 _stream(stream)), "attn_ceiling_fma")


def ceiling_exp2_fma(out, workgroups, iters, stream=None):
    """Enqueue the mixed probe: workgroups*256*iters*8 exponentials and 4x as many FMAs."""
    if out.numel() < workgroups * 256:
        raise ValueError("ceiling_exp2_fma: out too small")
    _probe_check(load_library().attn_ceiling_exp2_fma(_ptr(out), int(workgroups), int(iters),
                                                      _stream(stream)), "attn_ceiling_exp2_fma")


def ceiling_lds_read(out, workgroups, iters, transposed, stream=None):
    """Enqueue the LDS read probe: workgroups*512*iters*8 reads of 16 bytes
    (ds_read_b128) or 8 bytes (transposed: ds_read_b64_tr_b16)."""
    if out.numel() < workgroups * 512:
        raise ValueError("ceiling_lds_read: out too small")
    _probe_check(load_library().attn_ceiling_lds_read(_ptr(out), int(workgroups), int(iters),
                                                      int(bool(transposed)), _stream(stream)),
                 "attn_ceiling_lds_read")


def ceiling_copy(dst, src, stream=None):
    """Enqueue an HBM copy of src into dst (same byte size, a multiple of 16)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("ceiling_copy: dst and src sizes differ")
    _probe_check(load_library().attn_ceiling_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)),
                 "attn_ceiling_copy")
