"""Plain float64 CPU oracle for the attention forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or
links this package; only the tests, the package smoke check and the bench's
CPU-baseline leg use it. It shares no code with the HIP path.

What it computes (plain definition, full softmax materialised on purpose):

  For every batch b, head h, query row i, with g = h // (H // Hkv):
    s[i, j] = scale * sum_t q[b,h,i,t] * k[b,g,j,t]             j < Lk
    s[i, j] = -inf  where (causal and j > i) or (kv_len given and
                                              j >= clamp(kv_len[b], 0, Lk))
    p[i, j] = exp(s[i,j] - max_j s[i,j]) / sum_j exp(s[i,j] - max_j s[i,j])
    o[b,h,i,:] = sum_j p[i,j] * v[b,g,j,:]      (o = 0 when no key is valid)

Sources. The tutorial page "Guide de programmation pour la programmation GPU
par tuiles de NVIDIA : de cuTile et des noyaux Triton à Flash Attention"
(flash-attention paragraph and conclusion) fixes the operation: attention
checked against PyTorch's scaled-dot-product attention, which a tiled kernel
computes with an online softmax so the score matrix is never stored. This
oracle is that comparator's definition written out and does store it. The
broadcast variant follows "How We Built TLX" (Chinese translation, section
"Case study 2: in-kernel broadcast optimisation for RecSys"): candidate
queries read their user's keys/values at the users' own batch size, with no
replication; here that is q[c] attending over k[cand2user[c]],
v[cand2user[c]].

Jagged attention: the page "Meta 造了个 Triton 扩展 TLX ..." lists, among its
links, an article on jagged flash attention and gives nothing more. The plain
reading: B sequences packed token by token, q [total_q, H, d] and k, v
[total_kv, Hkv, d]; sequence b owns query tokens q_offsets[b] ..
q_offsets[b+1]-1 and key tokens kv_offsets[b] .. kv_offsets[b+1]-1, and is
the definition above applied to its own slices (causal top-left in local
indices; no keys gives zero rows).

Fixed-block sparse attention: the same page lists an article on a
fixed-block sparse self-attention kernel, again title only. The plain
reading: a boolean block mask [Hm, ceil(Lq/blk), ceil(Lk/blk)] (Hm = 1 shared
by all heads, or one per head) removes the key blocks a query block does not
attend to; key j is allowed for query i only where mask[h, i // blk,
j // blk] is set, on top of the causal and kv_len masks.

In-kernel broadcast linear layer: the same "How We Built TLX" section names
a linear-compression kernel sped up by splitting the matrix product and
fusing the broadcast, and gives no formula. The plain reading: one linear
layer over the concatenated features [x_user[cand2user[c]], x_cand[c]] with
weight w [N, K_u + K_c] (user columns first) and an optional bias; the
oracle computes it on the replicated features, the way it would be computed
without the optimisation. ikbo_user_partial is the user half of that
product plus the bias (the quantity computed once per user).

Normalisation fused into attention: the TLX pages say normalisation can be
fused into GEMM and attention kernels, saving a memory round trip, and list an
article on it by title. The plain reading for this path: RMS normalisation of
every query and key row over d with a gain vector each (q-norm and k-norm),
x / sqrt(mean(x^2) + eps) * gamma, before the attention above; values are not
normalised.

Readings where the pages are silent (each is also listed with the design
notes): scale defaults to 1/sqrt(d); the mask is additive -inf; causal is
top-left (key j allowed iff j <= i); kv_len is one value per K/V batch entry,
clamped to [0, Lk], masking keys only; a row with no valid key outputs 0; GQA
maps query head h to K/V head h // (H // Hkv); a candidate whose cand2user is
out of range gets NaN rows.

Parity pins: every function here is pinned by tests/test_oracle_pins.py
(closed forms, exact rational golden fixture, invariants, brute force in
40-digit decimal arithmetic, PyTorch float64 SDPA special cases) and
tests/test_oracle_mutants.py shows that plausible planted mistakes fail at
least one pin. No function is parity-unpinned.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["attention", "attention_rows", "attention_bcast", "attention_jagged",
           "attention_jagged_rows", "attention_block_sparse", "attention_block_sparse_rows",
           "probabilities", "ikbo_linear", "ikbo_user_partial", "rms_norm",
           "attention_qknorm", "attention_qknorm_rows"]


def _default_scale(d: int, scale) -> float:
    # Scale reading: 1/sqrt(d) unless the caller gives one; 0 also means default.
    if scale is None or scale == 0:
        return 1.0 / math.sqrt(d)
    return float(scale)


def _allowed(rows: np.ndarray, Lk: int, causal: bool, kv_len_b, block=None) -> np.ndarray:
    """Boolean [len(rows), Lk]: which (query i, key j) pairs are not masked.

    block = (mask [nQB, nKB], blk) additionally allows (i, j) only where
    mask[i // blk, j // blk] is set.
    """
    j = np.arange(Lk)[None, :]
    i = np.asarray(rows)[:, None]
    ok = np.ones((len(rows), Lk), dtype=bool)
    if kv_len_b is not None:
        n = min(max(int(kv_len_b), 0), Lk)
        ok &= j < n
    if causal:
        ok &= j <= i
    if block is not None:
        bm, blk = block
        ok &= np.asarray(bm, dtype=bool)[i // blk, j // blk]
    return ok


def _softmax_rows(s: np.ndarray, ok: np.ndarray) -> np.ndarray:
    """Row softmax of s over the allowed entries; rows with none give zeros."""
    if s.shape[1] == 0:                       # no keys at all: every row has none
        return np.zeros_like(s)
    s = np.where(ok, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(ok, np.exp(s - m), 0.0)
    z = e.sum(axis=1, keepdims=True)
    return np.divide(e, z, out=np.zeros_like(e), where=z > 0)


def _head_rows(q_bh, k_bg, v_bg, rows, causal, kv_len_b, scale, block=None):
    s = scale * (q_bh[rows] @ k_bg.T)          # [R, Lk] scores
    p = _softmax_rows(s, _allowed(rows, k_bg.shape[0], causal, kv_len_b, block))
    return p @ v_bg, p


def probabilities(q, k, v, *, causal=False, kv_len=None, scale=None, b=0, h=0):
    """The full softmax matrix P [Lq, Lk] of one (b, h); used by the invariant pins."""
    q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
    B, H, Lq, d = q.shape
    g = h // (H // k.shape[1])
    kvl = None if kv_len is None else kv_len[b]
    _, p = _head_rows(q[b, h], k[b, g], np.asarray(v, np.float64)[b, g], np.arange(Lq),
                      causal, kvl, _default_scale(d, scale))
    return p


def attention(q, k, v, *, causal=False, kv_len=None, scale=None):
    """Dense / causal / kv_len-masked / GQA attention forward, float64.

    q [B,H,Lq,d], k and v [B,Hkv,Lk,d] (any real dtype, widened exactly to
    float64), kv_len None or int array [B]. Returns o [B,H,Lq,d] float64.
    """
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    B, H, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    assert H % Hkv == 0 and k.shape == v.shape == (B, Hkv, Lk, d)
    group = H // Hkv
    sc = _default_scale(d, scale)
    o = np.zeros((B, H, Lq, d))
    rows = np.arange(Lq)
    for b in range(B):
        kvl = None if kv_len is None else kv_len[b]
        for h in range(H):
            g = h // group
            o[b, h], _ = _head_rows(q[b, h], k[b, g], v[b, g], rows, causal, kvl, sc)
    return o


def attention_rows(q, k, v, b, h, rows, *, causal=False, kv_len=None, scale=None):
    """Output rows o[b, h, rows, :] only (for sampled checks at full size)."""
    q_bh = np.asarray(q[b, h], np.float64)
    H, Hkv = q.shape[1], k.shape[1]
    g = h // (H // Hkv)
    k_bg, v_bg = np.asarray(k[b, g], np.float64), np.asarray(v[b, g], np.float64)
    kvl = None if kv_len is None else kv_len[b]
    out, _ = _head_rows(q_bh, k_bg, v_bg, np.asarray(rows), causal, kvl,
                        _default_scale(q.shape[3], scale))
    return out


def attention_bcast(q, k, v, cand2user, *, causal=False, kv_len=None, scale=None,
                    cands=None, rows=None):
    """In-kernel-broadcast attention: candidate c attends to user cand2user[c].

    q [B_c,H,Lq,d]; k, v [B_u,Hkv,Lk,d]; cand2user [B_c]; kv_len None or [B_u].
    Candidates whose user index is outside [0, B_u) get NaN rows.
    cands / rows optionally restrict the candidates and query rows computed;
    the result then has shape [len(cands), H, len(rows), d].
    """
    B_c, H, Lq, d = q.shape
    B_u, Hkv = k.shape[0], k.shape[1]
    group = H // Hkv
    sc = _default_scale(d, scale)
    cands = np.arange(B_c) if cands is None else np.asarray(cands)
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    o = np.zeros((len(cands), H, len(rows), d))
    for n, c in enumerate(cands):
        u = int(cand2user[c])
        if not 0 <= u < B_u:
            o[n] = np.nan
            continue
        kvl = None if kv_len is None else kv_len[u]
        for h in range(H):
            g = h // group
            o[n, h], _ = _head_rows(np.asarray(q[c, h], np.float64),
                                    np.asarray(k[u, g], np.float64),
                                    np.asarray(v[u, g], np.float64), rows, causal, kvl, sc)
    return o


def _seq_bounds(offsets, b):
    start = int(offsets[b])
    return start, max(int(offsets[b + 1]) - start, 0)


def attention_jagged(q, k, v, q_offsets, kv_offsets, *, causal=False, scale=None):
    """Jagged attention, float64: every sequence is the dense definition on its slices.

    q [total_q,H,d]; k, v [total_kv,Hkv,d]; q_offsets, kv_offsets int arrays
    [B+1]. Returns o [total_q,H,d] float64 (tokens outside every sequence: 0).
    """
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    H, d = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    assert H % Hkv == 0 and k.shape == v.shape and k.shape[2] == d
    group = H // Hkv
    sc = _default_scale(d, scale)
    o = np.zeros_like(q)
    for b in range(len(q_offsets) - 1):
        qs, lq = _seq_bounds(q_offsets, b)
        ks, lk = _seq_bounds(kv_offsets, b)
        rows = np.arange(lq)
        for h in range(H):
            g = h // group
            o[qs:qs + lq, h], _ = _head_rows(q[qs:qs + lq, h], k[ks:ks + lk, g],
                                             v[ks:ks + lk, g], rows, causal, None, sc)
    return o


def attention_jagged_rows(q, k, v, q_offsets, kv_offsets, b, h, rows, *, causal=False,
                          scale=None):
    """Rows `rows` (local to sequence b) of head h of the jagged output."""
    H, d, Hkv = q.shape[1], q.shape[2], k.shape[1]
    g = h // (H // Hkv)
    qs, _ = _seq_bounds(q_offsets, b)
    ks, lk = _seq_bounds(kv_offsets, b)
    rows = np.asarray(rows)
    q_bh = np.asarray(q[qs:qs + (int(rows.max()) + 1 if len(rows) else 0), h], np.float64)
    out, _ = _head_rows(q_bh, np.asarray(k[ks:ks + lk, g], np.float64),
                        np.asarray(v[ks:ks + lk, g], np.float64), rows, causal, None,
                        _default_scale(d, scale))
    return out


def _block_for_head(block_mask, blk, h):
    bm = np.asarray(block_mask)
    return (bm[0] if bm.shape[0] == 1 else bm[h]), int(blk)


def attention_block_sparse(q, k, v, block_mask, blk, *, causal=False, kv_len=None, scale=None):
    """Fixed-block sparse attention, float64: dense attention with key j allowed for
    query i only where block_mask[h, i // blk, j // blk] is set.

    q [B,H,Lq,d]; k, v [B,Hkv,Lk,d]; block_mask [1 or H, ceil(Lq/blk), ceil(Lk/blk)].
    """
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    B, H, Lq, d = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    group = H // Hkv
    sc = _default_scale(d, scale)
    o = np.zeros((B, H, Lq, d))
    rows = np.arange(Lq)
    for b in range(B):
        kvl = None if kv_len is None else kv_len[b]
        for h in range(H):
            g = h // group
            o[b, h], _ = _head_rows(q[b, h], k[b, g], v[b, g], rows, causal, kvl, sc,
                                    _block_for_head(block_mask, blk, h))
    return o


def attention_block_sparse_rows(q, k, v, block_mask, blk, b, h, rows, *, causal=False,
                                kv_len=None, scale=None):
    """Rows o[b, h, rows, :] of the block-sparse output (sampled checks at full size)."""
    H, Hkv = q.shape[1], k.shape[1]
    g = h // (H // Hkv)
    kvl = None if kv_len is None else kv_len[b]
    out, _ = _head_rows(np.asarray(q[b, h], np.float64), np.asarray(k[b, g], np.float64),
                        np.asarray(v[b, g], np.float64), np.asarray(rows), causal, kvl,
                        _default_scale(q.shape[3], scale), _block_for_head(block_mask, blk, h))
    return out


def ikbo_linear(x_user, x_cand, w, cand2user, bias=None):
    """In-kernel-broadcast linear layer, float64, written as the replicated product.

    x_user [B_u, K_u]; x_cand [B_c, K_c]; w [N, K_u + K_c], the weight of one
    linear layer over the concatenated features [user | candidate]; bias [N]
    or None; cand2user [B_c]. Returns y [B_c, N]:
        y[c] = concat(x_user[cand2user[c]], x_cand[c]) @ w.T + bias
    with NaN rows for candidates whose user index is outside [0, B_u).
    """
    xu, xc, w = (np.asarray(x, np.float64) for x in (x_user, x_cand, w))
    c2u = np.asarray(cand2user, np.int64)
    B_u, K_u = xu.shape
    B_c, K_c = xc.shape
    assert w.shape[1] == K_u + K_c and c2u.shape == (B_c,)
    bad = (c2u < 0) | (c2u >= B_u)
    u = np.where(bad, 0, c2u)
    rep = xu[u] if B_u > 0 else np.zeros((B_c, K_u))
    feats = np.concatenate([rep, xc], axis=1)
    y = feats @ w.T
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    y[bad] = np.nan
    return y


def ikbo_user_partial(x_user, w, bias=None):
    """The user half of the layer, once per user: z = x_user @ w[:, :K_u].T + bias."""
    xu, w = np.asarray(x_user, np.float64), np.asarray(w, np.float64)
    K_u = xu.shape[1]
    z = xu @ w[:, :K_u].T
    if bias is not None:
        z = z + np.asarray(bias, np.float64)[None, :]
    return z


def rms_norm(x, gamma=None, eps=1e-6):
    """Root-mean-square normalisation over the last axis, float64:
    x / sqrt(mean(x^2) + eps) * gamma (gamma None: ones)."""
    x = np.asarray(x, np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x * r
    if gamma is not None:
        y = y * np.asarray(gamma, np.float64)
    return y


def attention_qknorm(q, k, v, gamma_q=None, gamma_k=None, eps=1e-6, *, causal=False,
                     kv_len=None, scale=None):
    """Attention on RMS-normalised queries and keys: every row of q and of k is
    normalised over d (with its own gain vector), v is used as given."""
    return attention(rms_norm(q, gamma_q, eps), rms_norm(k, gamma_k, eps), v, causal=causal,
                     kv_len=kv_len, scale=scale)


def attention_qknorm_rows(q, k, v, b, h, rows, gamma_q=None, gamma_k=None, eps=1e-6, *,
                          causal=False, kv_len=None, scale=None):
    """Rows o[b, h, rows, :] of attention_qknorm (sampled checks at full size)."""
    H, Hkv = q.shape[1], k.shape[1]
    g = h // (H // Hkv)
    qn = rms_norm(q[b:b + 1, h:h + 1], gamma_q, eps)
    kn = rms_norm(k[b:b + 1, g:g + 1], gamma_k, eps)
    kvl = None if kv_len is None else np.asarray(kv_len)[b:b + 1]
    return attention_rows(qn, kn, np.asarray(v[b:b + 1, g:g + 1], np.float64), 0, 0, rows,
                          causal=causal, kv_len=kvl, scale=scale)
