"""Seeded synthetic inputs for the attention forward pass.

This module is shared by the oracle's tests, the GPU parity tests and the
bench. It holds none of the attention arithmetic: it only draws numbers,
rounds them to the storage type and converts storage types to float64.

Draws: numpy's Philox counter-based generator keyed by (seed, stream), so
every tensor has its own independent stream and the same numbers come out on
any machine with the same numpy. Normal samples are float32 N(0, 1); bf16
tensors are those samples rounded to nearest-even and held as raw uint16 bit
patterns.

Stream ids: Q=0, K=1, V=2, integers (kv_len) = 3, block masks = 4; the
linear layer's x_user=10, x_cand=11, w=12, bias=13, cand2user order=14; the
q/k norm gains 15 and row magnitudes 16.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import hashlib

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_INT = 0, 1, 2, 3
STREAM_XU, STREAM_XC, STREAM_W, STREAM_BIAS, STREAM_MAP = 10, 11, 12, 13, 14


def _gen(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.Philox(key=np.array([seed, stream], dtype=np.uint64)))


def normal_f32(shape, seed: int, stream: int) -> np.ndarray:
    """float32 N(0,1) samples of `shape` from stream (seed, stream)."""
    n = int(np.prod(shape))
    return _gen(seed, stream).standard_normal(n, dtype=np.float32).reshape(shape)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs here are finite normal samples, so NaN handling is not needed; an
    infinity stays an infinity.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a stored tensor ("bf16" bits or "f32")."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


@dataclass
class AttnInputs:
    """One attention problem. q/k/v are uint16 bf16 bits or float32 arrays.

    Dense:     q [B,H,Lq,d], k/v [B,Hkv,Lk,d], kv_len [B] or None.
    Broadcast: q [B_c,H,Lq,d], k/v [B_u,Hkv,Lk,d], cand2user [B_c],
               kv_len [B_u] or None.
    Jagged:    q [total_q,H,d], k/v [total_kv,Hkv,d], q_offsets and
               kv_offsets int32 [B+1].
    Block-sparse: dense q/k/v plus block_mask uint8 [1 or H, nQB, nKB] and blk.
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dtype: str
    causal: bool = False
    kv_len: np.ndarray | None = None
    cand2user: np.ndarray | None = None
    q_offsets: np.ndarray | None = None
    kv_offsets: np.ndarray | None = None
    block_mask: np.ndarray | None = None
    blk: int = 0
    gamma_q: np.ndarray | None = None   # q/k RMS-norm gains (float32 [d]), qknorm problems
    gamma_k: np.ndarray | None = None
    eps: float = 0.0
    scale: float | None = None
    meta: dict = field(default_factory=dict)

    def f64(self):
        return to_f64(self.q, self.dtype), to_f64(self.k, self.dtype), to_f64(self.v, self.dtype)


def _draw(shape, dtype, seed, stream):
    x = normal_f32(shape, seed, stream)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def make_dense(B, H, Hkv, Lq, Lk, d, *, dtype="bf16", causal=False, seed=0,
               kv_len_range=None, scale=None) -> AttnInputs:
    """Dense / causal / GQA / kv_len-masked problem with iid N(0,1) entries.

    kv_len_range=(lo, hi) draws kv_len[b] uniformly from the integers lo..hi
    inclusive on the integer stream.
    """
    q = _draw((B, H, Lq, d), dtype, seed, STREAM_Q)
    k = _draw((B, Hkv, Lk, d), dtype, seed, STREAM_K)
    v = _draw((B, Hkv, Lk, d), dtype, seed, STREAM_V)
    kv_len = None
    if kv_len_range is not None:
        lo, hi = kv_len_range
        kv_len = _gen(seed, STREAM_INT).integers(lo, hi + 1, size=B).astype(np.int32)
    return AttnInputs(q, k, v, dtype, causal=causal, kv_len=kv_len, scale=scale,
                      meta=dict(kind="dense", B=B, H=H, Hkv=Hkv, Lq=Lq, Lk=Lk, d=d))


def make_bcast(B_c, B_u, H, Hkv, Lq, Lk, d, *, dtype="bf16", causal=False, seed=0,
               cand2user=None, kv_len_range=None, scale=None, shuffle=False) -> AttnInputs:
    """Broadcast problem: B_c candidates' queries, B_u users' keys/values.

    cand2user defaults to the contiguous grouping c -> c // (B_c // B_u); shuffle=True
    permutes that map on its own stream (candidates of one user no longer adjacent).
    """
    q = _draw((B_c, H, Lq, d), dtype, seed, STREAM_Q)
    k = _draw((B_u, Hkv, Lk, d), dtype, seed, STREAM_K)
    v = _draw((B_u, Hkv, Lk, d), dtype, seed, STREAM_V)
    if cand2user is None:
        per = max(1, B_c // B_u)
        cand2user = np.minimum(np.arange(B_c) // per, B_u - 1)
        if shuffle:
            cand2user = _gen(seed, STREAM_MAP).permutation(cand2user)
    cand2user = np.asarray(cand2user, dtype=np.int32)
    kv_len = None
    if kv_len_range is not None:
        lo, hi = kv_len_range
        kv_len = _gen(seed, STREAM_INT).integers(lo, hi + 1, size=B_u).astype(np.int32)
    return AttnInputs(q, k, v, dtype, causal=causal, kv_len=kv_len, cand2user=cand2user,
                      scale=scale,
                      meta=dict(kind="bcast", B_c=B_c, B_u=B_u, H=H, Hkv=Hkv, Lq=Lq, Lk=Lk, d=d))


def make_jagged(B, H, Hkv, d, *, len_range=None, lengths=None, kv_lengths=None, dtype="bf16",
                causal=False, seed=0, scale=None) -> AttnInputs:
    """Jagged problem: B packed sequences with iid N(0,1) entries.

    Query lengths are `lengths`, or drawn uniformly from the integers
    len_range=(lo, hi) inclusive on the integer stream. Key lengths default to
    the query lengths (self-attention over each sequence).
    """
    if lengths is None:
        lo, hi = len_range
        lengths = _gen(seed, STREAM_INT).integers(lo, hi + 1, size=B)
    lengths = np.asarray(lengths, dtype=np.int64)
    kv_lengths = lengths if kv_lengths is None else np.asarray(kv_lengths, dtype=np.int64)
    q_offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    kv_offsets = np.concatenate([[0], np.cumsum(kv_lengths)]).astype(np.int32)
    q = _draw((int(q_offsets[-1]), H, d), dtype, seed, STREAM_Q)
    k = _draw((int(kv_offsets[-1]), Hkv, d), dtype, seed, STREAM_K)
    v = _draw((int(kv_offsets[-1]), Hkv, d), dtype, seed, STREAM_V)
    return AttnInputs(q, k, v, dtype, causal=causal, q_offsets=q_offsets, kv_offsets=kv_offsets,
                      scale=scale,
                      meta=dict(kind="jagged", B=B, H=H, Hkv=Hkv, d=d,
                                max_Lq=int(lengths.max(initial=0)),
                                max_Lk=int(kv_lengths.max(initial=0))))


def block_pattern(nqb: int, nkb: int, window: int, n_global: int) -> np.ndarray:
    """Fixed block pattern [1, nqb, nkb]: query block qb keeps key blocks
    qb-window+1 .. qb (a local band) and the first n_global key blocks."""
    qb = np.arange(nqb)[:, None]
    kb = np.arange(nkb)[None, :]
    keep = ((kb <= qb) & (kb > qb - window)) | (kb < n_global)
    return keep.astype(np.uint8)[None]


def make_block_sparse(B, H, Hkv, Lq, Lk, d, blk, *, dtype="bf16", causal=False, seed=0,
                      window=None, n_global=0, density=None, mask_heads=1,
                      kv_len_range=None, scale=None) -> AttnInputs:
    """Block-sparse problem: a dense problem plus a block mask, either the fixed
    local-window + global pattern (window given) or iid blocks kept with
    probability `density` drawn on the integer stream."""
    w = make_dense(B, H, Hkv, Lq, Lk, d, dtype=dtype, causal=causal, seed=seed,
                   kv_len_range=kv_len_range, scale=scale)
    nqb, nkb = -(-Lq // blk), -(-Lk // blk)
    if window is not None:
        mask = np.repeat(block_pattern(nqb, nkb, window, n_global), mask_heads, axis=0)
    else:
        r = _gen(seed, STREAM_INT + 1).random((mask_heads, nqb, nkb))
        mask = (r < density).astype(np.uint8)
    w.block_mask, w.blk = mask, blk
    w.meta = dict(kind="block_sparse", B=B, H=H, Hkv=Hkv, Lq=Lq, Lk=Lk, d=d, blk=blk,
                  mask_heads=mask_heads, window=window, n_global=n_global, density=density)
    return w


def make_qknorm(B, H, Hkv, Lq, Lk, d, *, causal=False, seed=0, kv_len_range=None, eps=1e-6,
                 scale=None, gains=True) -> AttnInputs:
    """A dense bf16 problem for attention on RMS-normalised queries and keys: q and k rows
    carry magnitudes 3 exp(0.5 N(0,1)) (so normalising matters), gains are
    1 + 0.2 N(0,1) (float32), v is N(0,1)."""
    rng = _gen(seed, STREAM_INT + 13)
    q = normal_f32((B, H, Lq, d), seed, STREAM_Q)
    k = normal_f32((B, Hkv, Lk, d), seed, STREAM_K)
    q *= np.float32(3.0) * np.exp(np.float32(0.5) * rng.standard_normal((B, H, Lq, 1))).astype(np.float32)
    k *= np.float32(3.0) * np.exp(np.float32(0.5) * rng.standard_normal((B, Hkv, Lk, 1))).astype(np.float32)
    v = _draw((B, Hkv, Lk, d), "bf16", seed, STREAM_V)
    kv_len = None
    if kv_len_range is not None:
        lo, hi = kv_len_range
        kv_len = _gen(seed, STREAM_INT).integers(lo, hi + 1, size=B).astype(np.int32)
    w = AttnInputs(f32_to_bf16_bits(q), f32_to_bf16_bits(k), v, "bf16", causal=causal,
                   kv_len=kv_len, scale=scale)
    if gains:
        g = _gen(seed, STREAM_INT + 12).standard_normal((2, d)).astype(np.float32)
        w.gamma_q = np.float32(1.0) + np.float32(0.2) * g[0]
        w.gamma_k = np.float32(1.0) + np.float32(0.2) * g[1]
    w.eps = float(eps)
    w.meta = dict(kind="qknorm", B=B, H=H, Hkv=Hkv, Lq=Lq, Lk=Lk, d=d, eps=float(eps))
    return w


# The workloads the method is measured on: tiny fp32 parity case, dense causal,
# in-kernel broadcast, kv_len-masked, long-sequence GQA causal, jagged causal
# self-attention over sequences of uniformly drawn lengths, and fixed-block
# sparse causal attention (a local band of 8 blocks plus 1 global block).
WORKLOADS = {
    "fp32_tiny": dict(kind="dense", B=1, H=1, Hkv=1, Lq=128, Lk=128, d=64, dtype="f32",
                      causal=False),
    "dense_causal_L2048": dict(kind="dense", B=4, H=16, Hkv=16, Lq=2048, Lk=2048, d=128,
                               dtype="bf16", causal=True),
    "bcast_Bc1024_Bu32": dict(kind="bcast", B_c=1024, B_u=32, H=8, Hkv=8, Lq=64, Lk=1024,
                              d=128, dtype="bf16", causal=False),
    # the same with the candidate -> user map shuffled (a user's candidates not adjacent)
    "bcast_Bc1024_Bu32_shuffled": dict(kind="bcast", B_c=1024, B_u=32, H=8, Hkv=8, Lq=64,
                                       Lk=1024, d=128, dtype="bf16", causal=False,
                                       shuffle=True),
    "masked_kvlen_L4096_d64": dict(kind="dense", B=8, H=16, Hkv=16, Lq=4096, Lk=4096, d=64,
                                   dtype="bf16", causal=False, kv_len_range=(2048, 4096)),
    "gqa_causal_L16384": dict(kind="dense", B=1, H=32, Hkv=8, Lq=16384, Lk=16384, d=128,
                              dtype="bf16", causal=True),
    "jagged_causal_B32": dict(kind="jagged", B=32, H=16, Hkv=16, d=128, len_range=(256, 4096),
                              dtype="bf16", causal=True),
    "block_sparse_L16384": dict(kind="block_sparse", B=1, H=16, Hkv=16, Lq=16384, Lk=16384,
                                d=128, blk=256, window=8, n_global=1, dtype="bf16",
                                causal=True),
    "qknorm_gqa_causal_L16384": dict(kind="qknorm", B=1, H=32, Hkv=8, Lq=16384, Lk=16384,
                                     d=128, dtype="bf16", causal=True),
}


def make_workload(name: str, seed: int = 0) -> AttnInputs:
    w = dict(WORKLOADS[name])
    kind = w.pop("kind")
    if kind == "dense":
        return make_dense(w.pop("B"), w.pop("H"), w.pop("Hkv"), w.pop("Lq"), w.pop("Lk"),
                          w.pop("d"), seed=seed, **w)
    if kind == "jagged":
        return make_jagged(w.pop("B"), w.pop("H"), w.pop("Hkv"), w.pop("d"), seed=seed, **w)
    if kind == "qknorm":
        w.pop("dtype")
        return make_qknorm(w.pop("B"), w.pop("H"), w.pop("Hkv"), w.pop("Lq"), w.pop("Lk"),
                           w.pop("d"), seed=seed, **w)
    if kind == "block_sparse":
        return make_block_sparse(w.pop("B"), w.pop("H"), w.pop("Hkv"), w.pop("Lq"), w.pop("Lk"),
                                 w.pop("d"), w.pop("blk"), seed=seed, **w)
    return make_bcast(w.pop("B_c"), w.pop("B_u"), w.pop("H"), w.pop("Hkv"), w.pop("Lq"),
                      w.pop("Lk"), w.pop("d"), seed=seed, **w)


@dataclass
class LinearInputs:
    """One in-kernel broadcast linear problem; x_user [B_u,K_u], x_cand [B_c,K_c] and
    w [N,K_u+K_c] are bf16 bits (uint16), bias float32 [N] or None, cand2user int32 [B_c]."""
    x_user: np.ndarray
    x_cand: np.ndarray
    w: np.ndarray
    bias: np.ndarray | None
    cand2user: np.ndarray
    out_dtype: str = "bf16"
    meta: dict = field(default_factory=dict)

    def f64(self):
        return (to_f64(self.x_user, "bf16"), to_f64(self.x_cand, "bf16"), to_f64(self.w, "bf16"),
                None if self.bias is None else self.bias.astype(np.float64))


def make_linear(B_u, B_c, K_u, K_c, N, *, bias=True, out_dtype="bf16", shuffle=False,
                cand2user=None, seed=0) -> LinearInputs:
    """Features iid N(0,1); weight N(0,1)/sqrt(K_u+K_c) (outputs of unit scale); bias
    0.1 N(0,1). cand2user defaults to contiguous groups of B_c // B_u candidates per
    user (the order in which one request's candidates arrive); shuffle=True permutes
    it on its own stream."""
    K = K_u + K_c
    x_user = f32_to_bf16_bits(normal_f32((B_u, K_u), seed, STREAM_XU))
    x_cand = f32_to_bf16_bits(normal_f32((B_c, K_c), seed, STREAM_XC))
    w = f32_to_bf16_bits(normal_f32((N, K), seed, STREAM_W) * np.float32(1.0 / np.sqrt(max(K, 1))))
    b = normal_f32((N,), seed, STREAM_BIAS) * np.float32(0.1) if bias else None
    if cand2user is None:
        per = max(1, B_c // max(B_u, 1))
        cand2user = np.minimum(np.arange(B_c) // per, max(B_u - 1, 0))
        if shuffle:
            cand2user = _gen(seed, STREAM_MAP).permutation(cand2user)
    cand2user = np.asarray(cand2user, dtype=np.int32)
    return LinearInputs(x_user, x_cand, w, b, cand2user, out_dtype,
                        meta=dict(kind="ikbo_linear", B_u=B_u, B_c=B_c, K_u=K_u, K_c=K_c, N=N,
                                  bias=bool(bias), out_dtype=out_dtype))


# The linear layer's workload: 2048 users with 32 candidates each, user
# features of 2048 and candidate features of 1024 compressed to 1024 outputs.
LINEAR_WORKLOADS = {
    "ikbo_linear_Bc65536": dict(B_u=2048, B_c=65536, K_u=2048, K_c=1024, N=1024, bias=True,
                                out_dtype="bf16"),
}


def make_linear_workload(name: str, seed: int = 0) -> LinearInputs:
    w = dict(LINEAR_WORKLOADS[name])
    return make_linear(w.pop("B_u"), w.pop("B_c"), w.pop("K_u"), w.pop("K_c"), w.pop("N"),
                       seed=seed, **w)
