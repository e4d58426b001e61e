"""Benchmark of the fused tiled attention forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-variants]
                [--no-cpu-baseline] [--no-ceiling] [--ceiling-only]

A step is one attention forward (one launch of the library's kernel) over the
workload's synthetic, seeded inputs, which are resident in HBM before timing
starts. Prints ONE JSON line. `value` is algorithmic TFLOP/s (4*d FLOPs per
unmasked query/key pair) of the headline workload, from HIP events around the
timed launches on the launch stream. `roofline` relates it to the bf16 MFMA
spec peak and to the peak the ceiling probes measure on the same GPU in the
same run (`frac_of_measured_peak`), warm (back-to-back launches) and cold
(`cold_ms_per_step`: median step time with L2 and the last-level cache
flushed by a 512 MiB write before each step). `ceiling` holds those probes:
MFMA with N(0,1) and constant operands, v_exp_f32, fp32 FMA, LDS reads and
an HBM copy. `cpu_baseline` times the float64 oracle on the host cores (one
thread per core of this job's share), over the whole workload where that
takes seconds and on a labelled sample otherwise. `variants` holds the other
workloads (the broadcast one also in GB/s), each with its own fractions, error
and CPU baseline, and the in-kernel broadcast linear layer (both of its
launches per step, 2 FLOPs per multiply-add of the decomposed products, with
torch's hipBLASLt products and gather on the same inputs timed beside it for
context). A step of the q/k-normalised workload is both of its launches (key
normalisation, then the attention pass with the query normalisation fused).
Each variant's timed steps follow at least 100 ms of untimed GPU work, so that
the clocks, which drop while the CPU baselines run, have ramped up again. The
shuffled broadcast variant is also timed through the grouped path (device
grouping of the candidates by user, then the attention with that packing).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import attn_inputs as ai  # noqa: E402

METRIC = "attention fwd TFLOP/s (bf16) and % of MFMA peak; broadcast-path GB/s"
HEADLINE = "gqa_causal_L16384"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense MFMA / fp32 matrix peaks
PEAK_HBM_GBS = 8000.0
# Untimed GPU time spent before each variant's timed steps (clock ramp after CPU work).
WARM_MS = 100.0
KERNEL_SOURCE = os.path.join(ROOT, "tiled_attention_attn_amd", "csrc", "attn_bf16.hip")
LINEAR_SOURCE = os.path.join(ROOT, "tiled_attention_attn_amd", "csrc", "ikbo_gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _seq_lengths(w: ai.AttnInputs):
    return np.diff(w.q_offsets).astype(np.int64), np.diff(w.kv_offsets).astype(np.int64)


def pairs(w: ai.AttnInputs) -> int:
    """Unmasked (query, key) pairs summed over batch entries (sequences) and heads."""
    if w.q_offsets is not None:
        H = w.q.shape[1]
        total = 0
        for lq, lk in zip(*_seq_lengths(w)):
            if w.causal:
                total += int(np.minimum(np.arange(lq) + 1, lk).sum())
            else:
                total += int(lq * lk)
        return total * H
    NB, H, Lq, _ = w.q.shape
    Lk = w.k.shape[2]
    if w.block_mask is not None:
        return _block_sparse_pairs(w)
    kv_b = w.kv_len if w.cand2user is None or w.kv_len is None else w.kv_len[w.cand2user]
    total = 0
    for b in range(NB):
        n = Lk if kv_b is None else int(min(max(kv_b[b], 0), Lk))
        if w.causal:
            i = np.arange(Lq)
            total += int(np.minimum(i + 1, n).sum())
        else:
            total += Lq * n
    return total * H


def _block_sparse_pairs(w: ai.AttnInputs) -> int:
    """Allowed (query, key) pairs under the block mask, causal and kv_len, all heads."""
    NB, H, Lq, _ = w.q.shape
    Lk, blk, bm = w.k.shape[2], w.blk, w.block_mask
    total = 0
    for b in range(NB):
        n = Lk if w.kv_len is None else int(min(max(w.kv_len[b], 0), Lk))
        for hm in range(bm.shape[0]):
            heads = H if bm.shape[0] == 1 else 1
            for qb in range(bm.shape[1]):
                i = np.arange(qb * blk, min((qb + 1) * blk, Lq))
                for kb in np.nonzero(bm[hm, qb])[0]:
                    lo, hi = kb * blk, min((kb + 1) * blk, n)
                    if hi <= lo:
                        continue
                    top = np.minimum(i + 1, hi) if w.causal else np.full(len(i), hi)
                    total += heads * int(np.maximum(top - lo, 0).sum())
    return total


def algorithmic_flops(w) -> int:
    return 4 * w.q.shape[-1] * pairs(w)


def algorithmic_bytes(w) -> int:
    """Read Q, the unique valid K/V rows and the index arrays; write O."""
    esz = 2 if w.dtype == "bf16" else 4
    if w.q_offsets is not None:   # jagged: every packed K/V token is read once
        return 2 * w.q.size * esz + 2 * w.k.size * esz + 4 * (w.q_offsets.size + w.kv_offsets.size)
    NKV, Hkv, Lk, d = w.k.shape
    if w.block_mask is not None:   # K/V blocks that some query block reads, plus the mask
        nkb = w.block_mask.shape[2]
        used = w.block_mask.any(axis=(0, 1))
        rows = sum(min((kb + 1) * w.blk, Lk) - kb * w.blk for kb in range(nkb) if used[kb])
        return 2 * w.q.size * esz + 2 * NKV * Hkv * rows * d * esz + w.block_mask.size
    kv_rows = 0
    for u in range(NKV):
        kv_rows += Lk if w.kv_len is None else int(min(max(w.kv_len[u], 0), Lk))
    total = 2 * w.q.size * esz + 2 * kv_rows * Hkv * d * esz
    for aux in (w.kv_len, w.cand2user):
        if aux is not None:
            total += 4 * aux.size
    return total


def kernel_source_hash(path: str = KERNEL_SOURCE) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def to_device(x: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


class Runner:
    def __init__(self, w: ai.AttnInputs, grouped: bool = False):
        import torch
        self.w = w
        # broadcast: group the candidates by user on the device every step, then run
        # the attention with that packing order (attn_bcast_group + attn_fwd_bcast_grouped)
        self.grouped = grouped and w.cand2user is not None
        self.q, self.k, self.v = (to_device(x, w.dtype) for x in (w.q, w.k, w.v))
        self.o = torch.empty_like(self.q)
        self.kv = None if w.kv_len is None else torch.from_numpy(w.kv_len).cuda()
        self.c2u = None if w.cand2user is None else torch.from_numpy(w.cand2user).cuda()
        self.qo = None if w.q_offsets is None else torch.from_numpy(w.q_offsets).cuda()
        self.ko = None if w.kv_offsets is None else torch.from_numpy(w.kv_offsets).cuda()
        self.bm = None if w.block_mask is None else torch.from_numpy(w.block_mask).cuda()
        self.qknorm = w.meta.get("kind") == "qknorm"
        if self.qknorm:
            self.gq = None if w.gamma_q is None else torch.from_numpy(w.gamma_q).cuda()
            self.gk = None if w.gamma_k is None else torch.from_numpy(w.gamma_k).cuda()
            self.kn = torch.empty_like(self.k)
        if self.grouped:
            self.order = torch.empty(w.cand2user.size, dtype=torch.int32, device="cuda")
            self.work = torch.empty(w.k.shape[0] + 1, dtype=torch.int32, device="cuda")
        import tiled_attention_attn_amd as taa
        self.taa = taa
        # Whether the library runs this problem on its 8-wave d = 128 schedule, whose
        # products use v_mfma_f32_16x16x32_bf16 (the library's rule: bf16, d = 128, at
        # least 4096 keys, block-sparse blocks a multiple of 256 rows, no override).
        m = w.meta
        lk = m.get("Lk", m.get("max_Lk", 0))
        forced = os.environ.get("ATTN_BF16_WAVES", "")
        self.m16 = (w.dtype == "bf16" and m.get("d") == 128 and
                    ((lk >= 4096 and forced in ("", "0")) or forced == "8") and
                    (w.block_mask is None or w.blk % 256 == 0))

    def __call__(self):
        if self.qknorm:
            self.taa.attn_fwd_qknorm(self.q, self.k, self.v, self.gq, self.gk, self.w.eps, self.o,
                                     self.kn, causal=self.w.causal, kv_len=self.kv)
        elif self.bm is not None:
            self.taa.attn_fwd_block_sparse(self.q, self.k, self.v, self.bm, self.w.blk, self.o,
                                           causal=self.w.causal, kv_len=self.kv)
        elif self.qo is not None:
            self.taa.attn_fwd_jagged(self.q, self.k, self.v, self.qo, self.ko,
                                     self.w.meta["max_Lq"], self.w.meta["max_Lk"], self.o,
                                     causal=self.w.causal)
        elif self.c2u is None:
            self.taa.attn_fwd(self.q, self.k, self.v, self.o, causal=self.w.causal,
                              kv_len=self.kv)
        elif self.grouped:
            self.taa.bcast_group(self.c2u, self.w.k.shape[0], self.order, work=self.work)
            self.taa.attn_fwd_bcast(self.q, self.k, self.v, self.c2u, self.o,
                                    causal=self.w.causal, kv_len=self.kv, order=self.order)
        else:
            self.taa.attn_fwd_bcast(self.q, self.k, self.v, self.c2u, self.o,
                                    causal=self.w.causal, kv_len=self.kv)


def time_steps(fn, steps: int, warmup: int, warm_ms: float = 0.0) -> float:
    """Average milliseconds per step, from HIP events on the launch stream. After the
    `warmup` steps, further untimed steps run until at least `warm_ms` of GPU time has
    been spent warming up: after seconds of CPU work (the oracle baselines) the GPU
    clocks are down, and a short timed region would otherwise start before they ramp."""
    import torch
    for _ in range(warmup):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    done = 0.0
    while done < warm_ms:
        a.record()
        for _ in range(4):
            fn()
        b.record()
        torch.cuda.synchronize()
        done += a.elapsed_time(b)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_cold(fn, reps: int = 10) -> float:
    """Median milliseconds of one step with cold caches: a 512 MiB write before each
    step evicts L2 and the last-level cache; only the step itself is timed."""
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps):
        flush.fill_(1)
        start.record()
        fn()
        end.record()
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end))
    del flush
    return float(np.median(times))


def sampled_error(run: Runner, seed: int = 1, nrows: int = 4) -> tuple[float, dict]:
    """Max abs error of a few output rows against the float64 oracle, and where it is
    (batch entry or sequence b, head h, query row, column)."""
    import oracle
    import torch
    w = run.w
    rng = np.random.default_rng(seed)
    if w.q_offsets is not None:
        return _sampled_error_jagged(run, rng, nrows)
    NB, H, Lq, _ = w.q.shape
    worst, where = 0.0, {}
    for _ in range(2):
        b, h = int(rng.integers(NB)), int(rng.integers(H))
        rows = np.unique(np.concatenate([[0, Lq - 1], rng.integers(0, Lq, nrows)]))
        got = run.o[b, h, torch.from_numpy(rows).cuda()].double().cpu().numpy()
        u = b if w.cand2user is None else int(w.cand2user[b])
        g = h // (H // w.k.shape[1])
        kvl = None if w.kv_len is None else w.kv_len[u:u + 1]
        qf, kf, vf = (ai.to_f64(x, w.dtype) for x in
                      (w.q[b:b + 1, h:h + 1], w.k[u:u + 1, g:g + 1], w.v[u:u + 1, g:g + 1]))
        if run.qknorm:
            ref = oracle.attention_qknorm_rows(qf, kf, vf, 0, 0, rows, w.gamma_q, w.gamma_k,
                                               w.eps, causal=w.causal, kv_len=kvl)
        elif w.block_mask is not None:
            bm = w.block_mask[0:1] if w.block_mask.shape[0] == 1 else w.block_mask[h:h + 1]
            ref = oracle.attention_block_sparse_rows(qf, kf, vf, bm, w.blk, 0, 0, rows,
                                                     causal=w.causal, kv_len=kvl)
        else:
            ref = oracle.attention_rows(qf, kf, vf, 0, 0, rows, causal=w.causal, kv_len=kvl)
        err = np.abs(got - ref)
        i, j = np.unravel_index(int(np.argmax(err)), err.shape)
        if err[i, j] >= worst:
            worst = float(err[i, j])
            where = {"b": b, "h": h, "row": int(rows[i]), "col": int(j)}
    return worst, where


def _sampled_error_jagged(run: Runner, rng, nrows: int) -> tuple[float, dict]:
    import oracle
    import torch
    w = run.w
    H, Hkv = w.q.shape[1], w.k.shape[1]
    worst, where = 0.0, {}
    for _ in range(2):
        b, h = int(rng.integers(len(w.q_offsets) - 1)), int(rng.integers(H))
        qs, qe = int(w.q_offsets[b]), int(w.q_offsets[b + 1])
        ks, ke = int(w.kv_offsets[b]), int(w.kv_offsets[b + 1])
        if qe == qs:
            continue
        rows = np.unique(np.concatenate([[0, qe - qs - 1], rng.integers(0, qe - qs, nrows)]))
        got = run.o[torch.from_numpy(qs + rows).cuda(), h].double().cpu().numpy()
        g = h // (H // Hkv)
        ref = oracle.attention_jagged_rows(
            ai.to_f64(w.q[qs:qe, h:h + 1], w.dtype), ai.to_f64(w.k[ks:ke, g:g + 1], w.dtype),
            ai.to_f64(w.v[ks:ke, g:g + 1], w.dtype), [0, qe - qs], [0, ke - ks], 0, 0, rows,
            causal=w.causal)
        err = np.abs(got - ref)
        i, j = np.unravel_index(int(np.argmax(err)), err.shape)
        if err[i, j] >= worst:
            worst = float(err[i, j])
            where = {"b": b, "h": h, "row": int(rows[i]), "col": int(j)}
    return worst, where


def oracle_threads() -> tuple[int, int]:
    """(threads the oracle runs on, cores in this process's affinity set). The threads are
    the affinity set, capped by OMP_NUM_THREADS when it is set (this job's share of the
    host's cores)."""
    aff = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = min(aff, int(env)) if env.isdigit() and int(env) > 0 else aff
    return max(1, n), aff


def _units(w: ai.AttnInputs):
    """(batch entry or sequence, head) pairs of a workload with their query-row counts."""
    if w.q_offsets is not None:
        lq = np.diff(w.q_offsets)
        return [(b, h, int(lq[b])) for b in range(len(lq)) for h in range(w.q.shape[1])
                if lq[b] > 0]
    NB, H, Lq, _ = w.q.shape
    return [(b, h, Lq) for b in range(NB) for h in range(H)]


def _allowed_pairs(w: ai.AttnInputs, b: int, h: int, rows: np.ndarray) -> int:
    """Unmasked (query, key) pairs of the given query rows of (b, h)."""
    if w.q_offsets is not None:
        lk = int(np.diff(w.kv_offsets)[b])
        return int((np.minimum(rows + 1, lk) if w.causal else np.full(len(rows), lk)).sum())
    Lk = w.k.shape[2]
    u = b if w.cand2user is None else int(w.cand2user[b])
    n = Lk if w.kv_len is None else int(min(max(w.kv_len[u], 0), Lk))
    top = np.minimum(rows + 1, n) if w.causal else np.full(len(rows), n)
    if w.block_mask is None:
        return int(top.sum())
    bm = w.block_mask[0 if w.block_mask.shape[0] == 1 else h]
    total = 0
    for kb in range(bm.shape[1]):
        lo, hi = kb * w.blk, min((kb + 1) * w.blk, n)
        on = bm[rows // w.blk, kb] != 0
        total += int(np.maximum(np.minimum(top, hi) - lo, 0)[on].sum())
    return total


def _oracle_unit(w: ai.AttnInputs, b: int, h: int, rows) -> int:
    """The oracle as it stands on one (batch entry or sequence b, head h): every query row
    (rows None) or the given ones. Returns the algorithmic FLOPs of those rows (4 d per
    unmasked pair), which is what the GPU is credited with for the same rows."""
    import oracle
    d = w.q.shape[-1]
    if w.q_offsets is not None:
        H, Hkv = w.q.shape[1], w.k.shape[1]
        g = h // (H // Hkv)
        qs, qe = int(w.q_offsets[b]), int(w.q_offsets[b + 1])
        ks, ke = int(w.kv_offsets[b]), int(w.kv_offsets[b + 1])
        qf, kf, vf = (ai.to_f64(x, w.dtype) for x in
                      (w.q[qs:qe, h:h + 1], w.k[ks:ke, g:g + 1], w.v[ks:ke, g:g + 1]))
        if rows is None:
            oracle.attention_jagged(qf, kf, vf, [0, qe - qs], [0, ke - ks], causal=w.causal,
                                    scale=w.scale)
            rows = np.arange(qe - qs)
        else:
            oracle.attention_jagged_rows(qf, kf, vf, [0, qe - qs], [0, ke - ks], 0, 0, rows,
                                         causal=w.causal, scale=w.scale)
        return 4 * d * _allowed_pairs(w, b, h, rows)
    H, Hkv = w.q.shape[1], w.k.shape[1]
    g = h // (H // Hkv)
    u = b if w.cand2user is None else int(w.cand2user[b])
    qf, kf, vf = (ai.to_f64(x, w.dtype) for x in
                  (w.q[b:b + 1, h:h + 1], w.k[u:u + 1, g:g + 1], w.v[u:u + 1, g:g + 1]))
    kvl = None if w.kv_len is None else w.kv_len[u:u + 1]
    if w.meta.get("kind") == "qknorm":
        if rows is None:
            oracle.attention_qknorm(qf, kf, vf, w.gamma_q, w.gamma_k, w.eps, causal=w.causal,
                                    kv_len=kvl, scale=w.scale)
        else:
            oracle.attention_qknorm_rows(qf, kf, vf, 0, 0, rows, w.gamma_q, w.gamma_k, w.eps,
                                         causal=w.causal, kv_len=kvl, scale=w.scale)
    elif w.block_mask is not None:
        bm = w.block_mask[0:1] if w.block_mask.shape[0] == 1 else w.block_mask[h:h + 1]
        if rows is None:
            oracle.attention_block_sparse(qf, kf, vf, bm, w.blk, causal=w.causal, kv_len=kvl,
                                          scale=w.scale)
        else:
            oracle.attention_block_sparse_rows(qf, kf, vf, bm, w.blk, 0, 0, rows,
                                               causal=w.causal, kv_len=kvl, scale=w.scale)
    elif rows is None:
        oracle.attention(qf, kf, vf, causal=w.causal, kv_len=kvl, scale=w.scale)
    else:
        oracle.attention_rows(qf, kf, vf, 0, 0, rows, causal=w.causal, kv_len=kvl,
                              scale=w.scale)
    if rows is None:
        rows = np.arange(w.q.shape[2])
    return 4 * d * _allowed_pairs(w, b, h, rows)


def cpu_baseline(w: ai.AttnInputs, full: bool, budget_s: float = 15.0) -> dict:
    """Time the float64 oracle, as it stands, on the host cores: one thread per core of
    this job's share (see oracle_threads), each running the oracle on one (batch entry or
    sequence, head) at a time, with the BLAS inside each call single-threaded.

    full: every (b, h) pair and every query row, the whole workload. Otherwise a bounded
    sample: random pairs with up to 256 random query rows each (so causal and kv_len
    masking weigh in as in the whole workload), submitted until `budget_s` of wall time
    is spent. The oracle computes each sampled row's full score row, masked keys
    included; only unmasked pairs count as FLOPs, as on the GPU."""
    import concurrent.futures as cf
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        blas_one = threadpool_limits(1)
    except Exception:
        blas_one = contextlib.nullcontext()
    threads, aff = oracle_threads()
    units = _units(w)
    rng = np.random.default_rng(123)
    flops, done = 0, 0
    t0 = time.perf_counter()
    with blas_one, cf.ThreadPoolExecutor(threads) as ex:
        if full:
            for f in ex.map(lambda u: _oracle_unit(w, u[0], u[1], None), units):
                flops += f
            done = len(units)
        else:
            order = rng.permutation(len(units))
            pending, i = set(), 0
            while True:
                while len(pending) < threads and time.perf_counter() - t0 < budget_s:
                    b, h, L = units[order[i % len(units)]]
                    i += 1
                    rows = np.sort(rng.choice(L, size=min(256, L), replace=False))
                    pending.add(ex.submit(_oracle_unit, w, b, h, rows))
                if not pending:
                    break
                finished, pending = cf.wait(pending, return_when=cf.FIRST_COMPLETED)
                for f in finished:
                    flops += f.result()
                    done += 1
    wall = time.perf_counter() - t0
    unit_name = "(sequence, head)" if w.q_offsets is not None else "(batch entry, head)"
    what = {k: v for k, v in w.meta.items() if k != "kind"}
    if full:
        sample = (f"the whole workload: all {done} {unit_name} pairs, every query row "
                  f"({flops:.3e} algorithmic FLOPs in {wall:.1f} s) of {what}")
    else:
        sample = (f"sampled: {done} random {unit_name} pairs x up to 256 random query rows "
                  f"({flops:.3e} algorithmic FLOPs in {wall:.1f} s) of {what}")
    return {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": threads,
            "affinity_cores": aff, "kind": "oracle", "full": bool(full),
            "seconds": round(wall, 2), "sample": sample}


# Workloads whose whole oracle run stays within seconds on the host: the CPU baseline
# runs them in full; the others (the oracle materialises every score row, about
# 4.4 TFLOP of fp64 work on the L=16384 shapes) are sampled.
CPU_FULL = {"fp32_tiny", "dense_causal_L2048", "bcast_Bc1024_Bu32", "bcast_Bc1024_Bu32_shuffled",
            "masked_kvlen_L4096_d64"}


def linear_variant(name: str, steps: int, warmup: int = 3, warm_ms: float = WARM_MS) -> dict:
    """Time the in-kernel broadcast linear layer on its workload (both launches: the
    user half, then the candidate half with the gathered user rows), with sampled
    rows checked against the float64 oracle."""
    import oracle
    import torch
    import tiled_attention_attn_amd as taa
    wl = ai.make_linear_workload(name, seed=0)
    B_u, K_u = wl.x_user.shape
    B_c, K_c = wl.x_cand.shape
    N = wl.w.shape[0]
    xu, xc, w = (to_device(x, "bf16") for x in (wl.x_user, wl.x_cand, wl.w))
    bias = None if wl.bias is None else torch.from_numpy(wl.bias).cuda()
    c2u = torch.from_numpy(wl.cand2user).cuda()
    y = torch.empty((B_c, N), dtype=torch.bfloat16, device="cuda")
    z = torch.empty((B_u, N), dtype=torch.float32, device="cuda")
    step = lambda: taa.ikbo_linear(xu, xc, w, c2u, bias, y, z)  # noqa: E731
    ms = time_steps(step, steps, warmup, warm_ms=warm_ms)
    ms_cold = time_cold(step)
    flops = 2 * (B_u * K_u + B_c * K_c) * N
    nbytes = (2 * (wl.x_user.size + wl.x_cand.size + wl.w.size) + 4 * N + 4 * B_c
              + 2 * B_c * N + 2 * 4 * B_u * N)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, B_c - 1], rng.integers(0, B_c, 30)]))
    got = y[torch.from_numpy(rows).cuda()].double().cpu().numpy()
    xuf, _, wf, bf = wl.f64()
    ref = oracle.ikbo_linear(xuf, ai.to_f64(wl.x_cand[rows], "bf16"), wf, wl.cand2user[rows], bf)
    # The same computation through torch: hipBLASLt products and a torch gather.
    wu_t, wc_t = w[:, :K_u].t().contiguous(), w[:, K_u:].t().contiguous()
    c2u_l = c2u.long()
    bias_t = torch.zeros(N, device="cuda") if bias is None else bias
    ms_torch = time_steps(
        lambda: torch.mm(xc, wc_t) + (torch.mm(xu, wu_t).float() + bias_t)[c2u_l].bfloat16(),
        max(5, steps // 2), 3, warm_ms=warm_ms)
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms_per_step": round(ms, 5), "cold_ms_per_step": round(ms_cold, 5),
            "TFLOP/s": round(tf, 3),
            "frac_of_peak": round(tf / PEAK_TFLOPS["bf16"], 4), "dtype": "bf16",
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "algorithmic_flops_per_step": flops, "algorithmic_bytes_per_step": nbytes,
            "replication_equivalent_TFLOP/s":
                round(2 * B_c * (K_u + K_c) * N / (ms * 1e-3) / 1e12, 3),
            "torch_hipblaslt_decomposed_ms": round(ms_torch, 5),
            "max_abs_err_sampled": float(np.abs(got - ref).max()),
            "max_abs_err_sampled_at": {"candidate": int(rows[np.unravel_index(
                int(np.argmax(np.abs(got - ref))), got.shape)[0]]),
                "col": int(np.unravel_index(int(np.argmax(np.abs(got - ref))), got.shape)[1])},
            "config": dict(wl.meta)}


def linear_main(args) -> None:
    """The linear layer as the measured workload: one JSON line, as for attention."""
    ent = linear_variant(args.workload, args.steps, warmup=args.warmup, warm_ms=0.0)
    cfg = ent.pop("config")
    tf = ent["TFLOP/s"]
    out = {
        "metric": "in-kernel broadcast linear layer TFLOP/s (bf16, decomposed FLOPs)",
        "value": tf, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ent["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), Philox streams)",
        "config": {"workload": args.workload, **{k: v for k, v in cfg.items() if k != "kind"}},
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_TFLOPS["bf16"], 4),
                     "traffic": traffic_for(args.workload), "scope": "both launches of one step",
                     "algorithmic_flops_per_launch": ent["algorithmic_flops_per_step"],
                     "algorithmic_bytes_per_launch": ent["algorithmic_bytes_per_step"]},
        "max_abs_err_sampled": ent["max_abs_err_sampled"],
        "cold_ms_per_step": ent["cold_ms_per_step"],
        "replication_equivalent_TFLOP/s": ent["replication_equivalent_TFLOP/s"],
        "torch_hipblaslt_decomposed_ms": ent["torch_hipblaslt_decomposed_ms"],
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = linear_cpu_baseline(args.workload)
    print(json.dumps(out))


def linear_cpu_baseline(name: str, budget_s: float = 10.0) -> dict:
    """The float64 oracle, as it stands (replicated features), on random batches of 256
    candidates, one batch per thread of this job's share of the host cores (BLAS inside
    each call single-threaded), submitted until `budget_s` of wall time is spent; scaled
    to the layer's decomposed FLOPs per candidate, the unit the GPU is credited in."""
    import concurrent.futures as cf
    import contextlib
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        blas_one = threadpool_limits(1)
    except Exception:
        blas_one = contextlib.nullcontext()
    threads, aff = oracle_threads()
    wl = ai.make_linear_workload(name, seed=0)
    B_u, K_u = wl.x_user.shape
    B_c, K_c = wl.x_cand.shape
    N = wl.w.shape[0]
    xuf, _, wf, bf = wl.f64()
    per_cand = 2 * (B_u * K_u + B_c * K_c) * N / B_c
    rng = np.random.default_rng(123)

    def batch(rows):
        oracle.ikbo_linear(xuf, ai.to_f64(wl.x_cand[rows], "bf16"), wf, wl.cand2user[rows], bf)
        return len(rows)

    done = 0
    t0 = time.perf_counter()
    with blas_one, cf.ThreadPoolExecutor(threads) as ex:
        pending = set()
        while True:
            while len(pending) < threads and time.perf_counter() - t0 < budget_s:
                pending.add(ex.submit(batch, np.sort(rng.choice(B_c, size=256, replace=False))))
            if not pending:
                break
            finished, pending = cf.wait(pending, return_when=cf.FIRST_COMPLETED)
            done += sum(f.result() for f in finished)
    wall = time.perf_counter() - t0
    return {"value": per_cand * done / wall / 1e12, "unit": "TFLOP/s", "cores": threads,
            "affinity_cores": aff, "kind": "oracle", "full": False, "seconds": round(wall, 2),
            "sample": f"sampled: {done} random candidates of {B_c} in batches of 256 "
                      f"({wall:.1f} s), scaled to the layer's {per_cand:.4g} decomposed "
                      f"FLOPs per candidate"}


def ceiling(reps: int = 3) -> dict:
    """Sustained rates of the units the kernels use, measured on this GPU (median of
    `reps` timed launches after one warm launch, HIP events on the launch stream):
    bf16 MFMA from registers with N(0,1) operands (what attention inputs look like to
    the matrix cores) and with constant operands, v_exp_f32, scalar fp32 FMA, LDS reads
    (plain 16-byte and the transposing 8-byte form) and an HBM copy."""
    import torch
    from tiled_attention_attn_amd import _binding as b
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn) -> float:
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            start.record()
            fn()
            end.record()
            torch.cuda.synchronize()
            ts.append(start.elapsed_time(end))
        return float(np.median(ts))

    out = {}
    lanes = 65536
    ops_n = to_device(ai.f32_to_bf16_bits(ai.normal_f32((lanes * 128,), 0, 20)), "bf16")
    ops_c = torch.full((lanes * 128,), 1.0, dtype=torch.bfloat16, device="cuda")
    wg, waves, iters = 512, 8, 40000
    sink = torch.empty(wg * waves * 64, dtype=torch.float32, device="cuda")
    flops = wg * waves * iters * 8 * 32768
    for name, probe, ops in (("mfma_bf16_normal_operands", b.ceiling_mfma_bf16, ops_n),
                             ("mfma_bf16_constant_operands", b.ceiling_mfma_bf16, ops_c),
                             ("mfma16_bf16_normal_operands", b.ceiling_mfma16_bf16, ops_n)):
        ms = timed(lambda: probe(ops, sink, wg, waves, iters))
        tf = flops / (ms * 1e-3) / 1e12
        out[name] = {"TFLOP/s": round(tf, 1), "frac_of_spec": round(tf / PEAK_TFLOPS["bf16"], 4),
                     "ms": round(ms, 3)}
    del ops_n, ops_c, sink
    wg = 2048
    sink = torch.empty(wg * 512, dtype=torch.float32, device="cuda")
    iters = 20000
    ms = timed(lambda: b.ceiling_exp2(sink, wg, iters))
    n = wg * 256 * iters * 16
    exp_per_ms = n / ms
    out["v_exp_f32"] = {"G/s": round(n / (ms * 1e-3) / 1e9, 1),
                        "per_CU_per_clk_at_2.4GHz": round(n / (ms * 1e-3) / 256 / 2.4e9, 2),
                        "ms": round(ms, 3)}
    iters = 65536
    ms = timed(lambda: b.ceiling_fma(sink, wg, iters))
    n = wg * 256 * iters * 16
    fma_per_ms = n / ms
    out["v_fma_f32"] = {"TFLOP/s": round(2 * n / (ms * 1e-3) / 1e12, 2),
                        "per_CU_per_clk_at_2.4GHz": round(n / (ms * 1e-3) / 256 / 2.4e9, 2),
                        "ms": round(ms, 3)}
    # One exponential between every four FMAs, against the time each part takes alone
    # at the rates above: about 1 of their sum if the exponential takes FMA issue
    # slots, about 1 of the larger part if it runs beside them.
    iters = 16384
    ms = timed(lambda: b.ceiling_exp2_fma(sink, wg, iters))
    t_exp = wg * 256 * iters * 8 / exp_per_ms
    t_fma = wg * 256 * iters * 32 / fma_per_ms
    out["v_exp_f32_between_fmas"] = {"ms": round(ms, 3), "exp_part_alone_ms": round(t_exp, 3),
                                     "fma_part_alone_ms": round(t_fma, 3),
                                     "over_sum_of_parts": round(ms / (t_exp + t_fma), 3),
                                     "over_larger_part": round(ms / max(t_exp, t_fma), 3)}
    wg, iters = 512, 32768
    for name, tr, nb in (("lds_read_b128", 0, 16), ("lds_read_b64_tr_b16", 1, 8)):
        ms = timed(lambda: b.ceiling_lds_read(sink, wg, iters, tr))
        by = wg * 512 * iters * 8 * nb
        out[name] = {"TB/s": round(by / (ms * 1e-3) / 1e12, 2),
                     "B_per_CU_per_clk_at_2.4GHz": round(by / (ms * 1e-3) / 256 / 2.4e9, 1),
                     "ms": round(ms, 3)}
    del sink
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms = timed(lambda: b.ceiling_copy(dst, src))
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    out["hbm_copy"] = {"GB/s": round(gbs, 1), "frac_of_spec": round(gbs / PEAK_HBM_GBS, 4),
                       "bytes_copied": nbytes, "ms": round(ms, 3)}
    del src, dst
    torch.cuda.empty_cache()
    return out


def traffic_for(workload: str):
    """HBM bytes per launch (per step for the linear layer) measured with rocprofv3
    counters, if they were taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    ent = rec.get(workload)
    src = LINEAR_SOURCE if workload in ai.LINEAR_WORKLOADS else KERNEL_SOURCE
    if not ent or ent.get("kernel_source_sha256_16") != kernel_source_hash(src):
        return None
    return ent.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default=HEADLINE,
                    choices=sorted(ai.WORKLOADS) + sorted(ai.LINEAR_WORKLOADS))
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the ceiling microbenchmarks (and the measured-peak fractions)")
    ap.add_argument("--ceiling-only", action="store_true",
                    help="only run the ceiling microbenchmarks and print their JSON")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the "
              "method runs on one GPU's share; see the sharding notes in the design).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a visible MI355X GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "copies": 5}))
        return

    if args.ceiling_only:
        print(json.dumps({"ceiling": ceiling()}))
        return

    if args.workload in ai.LINEAR_WORKLOADS:
        linear_main(args)
        return
    w = ai.make_workload(args.workload, seed=0)
    run = Runner(w)
    ms = time_steps(run, args.steps, args.warmup)
    ms_cold = time_cold(run)
    flops = algorithmic_flops(w)
    nbytes = algorithmic_bytes(w)
    tflops = flops / (ms * 1e-3) / 1e12
    tf_cold = flops / (ms_cold * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    err, err_at = sampled_error(run)
    traffic = traffic_for(args.workload)
    m16 = run.m16
    del run
    torch.cuda.empty_cache()
    ceil = None if args.no_ceiling else ceiling()
    # the probe of the matrix-core shape the measured kernel runs (16 x 16 x 32 for
    # the 8-wave d = 128 schedule, 32 x 32 x 16 otherwise)
    probe = "mfma16_bf16_normal_operands" if m16 else "mfma_bf16_normal_operands"
    measured = None if ceil is None else ceil[probe]["TFLOP/s"]
    roofline = {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tflops / peak, 4), "traffic": traffic,
                "achieved_cold": round(tf_cold, 3), "frac_cold": round(tf_cold / peak, 4),
                "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes}
    if measured and w.dtype == "bf16":
        roofline.update({
            "measured_peak": measured,
            "measured_peak_source": f"ceiling.{probe}: "
                                    + ("v_mfma_f32_16x16x32_bf16" if m16 else "v_mfma_f32_32x32x16_bf16")
                                    + " from registers, N(0,1) operands, this GPU, this run",
            "frac_of_measured_peak": round(tflops / measured, 4),
            "frac_cold_of_measured_peak": round(tf_cold / measured, 4)})
    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), Philox streams)",
        "config": {"workload": args.workload, **{k: v for k, v in w.meta.items() if k != "kind"},
                   "causal": w.causal},
        "roofline": roofline,
        "max_abs_err_sampled": err,
        "max_abs_err_sampled_at": err_at,
        "cold_ms_per_step": round(ms_cold, 5),
    }
    if ceil is not None:
        out["ceiling"] = ceil
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.workload in CPU_FULL)
    if not args.no_variants:
        variants = {}
        for name in sorted(ai.WORKLOADS):
            if name == args.workload:
                continue
            wv = ai.make_workload(name, seed=0)
            rv = Runner(wv)
            msv = time_steps(rv, max(5, args.steps // 2), 3, warm_ms=WARM_MS)
            msc = time_cold(rv, 5)
            fv, bv = algorithmic_flops(wv), algorithmic_bytes(wv)
            tv = fv / (msv * 1e-3) / 1e12
            ev, ev_at = sampled_error(rv)
            ent = {"ms_per_step": round(msv, 5), "cold_ms_per_step": round(msc, 5),
                   "TFLOP/s": round(tv, 3),
                   "frac_of_peak": round(tv / PEAK_TFLOPS[wv.dtype], 4),
                   "frac_cold_of_peak": round(fv / (msc * 1e-3) / 1e12 / PEAK_TFLOPS[wv.dtype], 4),
                   "dtype": wv.dtype, "GB/s": round(bv / (msv * 1e-3) / 1e9, 1),
                   "max_abs_err_sampled": ev, "max_abs_err_sampled_at": ev_at}
            if measured and wv.dtype == "bf16":
                ent["frac_of_measured_peak"] = round(tv / measured, 4)
            if wv.cand2user is not None and name.endswith("_shuffled"):
                # the same inputs through the grouped path (grouping included in each step)
                rg = Runner(wv, grouped=True)
                msg = time_steps(rg, max(5, args.steps // 2), 3, warm_ms=WARM_MS)
                eg, eg_at = sampled_error(rg)
                ent["grouped"] = {"ms_per_step": round(msg, 5),
                                  "TFLOP/s": round(fv / (msg * 1e-3) / 1e12, 3),
                                  "max_abs_err_sampled": eg, "max_abs_err_sampled_at": eg_at,
                                  "path": "attn_bcast_group + attn_fwd_bcast_grouped per step"}
                del rg
            if wv.cand2user is not None:
                ent["GB/s_frac_of_hbm"] = round(ent["GB/s"] / PEAK_HBM_GBS, 4)
                rep = 2 * wv.q.size * 2 + 2 * wv.cand2user.size * wv.k[0].size * 2
                ent["replication_equivalent_GB/s"] = round(rep / (msv * 1e-3) / 1e9, 1)
            del rv
            torch.cuda.empty_cache()
            if not args.no_cpu_baseline:
                ent["cpu_baseline"] = cpu_baseline(wv, name in CPU_FULL, budget_s=5.0)
            variants[name] = ent
        for name in sorted(ai.LINEAR_WORKLOADS):
            ent = linear_variant(name, max(5, args.steps // 2))
            if measured:
                ent["frac_of_measured_peak"] = round(ent["TFLOP/s"] / measured, 4)
            if not args.no_cpu_baseline:
                ent["cpu_baseline"] = linear_cpu_baseline(name, budget_s=5.0)
            variants[name] = ent
            torch.cuda.empty_cache()
        out["variants"] = variants
    print(json.dumps(out))


if __name__ == "__main__":
    main()
