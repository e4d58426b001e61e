/*
 * attn.h - C ABI of the MI355X (gfx950) fused tiled attention forward pass
 * and the in-kernel broadcast linear layer.
 *
 * Operation. For every batch entry b, query head h and query row i,
 *     O[b,h,i,:] = sum_j softmax_j( scale * <Q[b,h,i,:], K[b,g,j,:]> + mask[i,j] ) * V[b,g,j,:]
 * with g = h / (H / Hkv) (grouped-query heads: contiguous groups of H/Hkv
 * query heads share one K/V head). The tutorial page "Guide de programmation
 * pour la programmation GPU par tuiles de NVIDIA : de cuTile et des noyaux
 * Triton a Flash Attention" (flash-attention paragraph and conclusion) gives
 * the method: attention computed tile by tile with an online softmax so the
 * Lq x Lk score matrix is never materialised, checked against PyTorch's
 * scaled-dot-product attention. The in-kernel broadcast variant follows "How
 * We Built TLX" (Chinese translation, "Case study 2: in-kernel broadcast
 * optimisation for RecSys"): candidates and users arrive at their own batch
 * sizes and the kernel reads each candidate's user K/V through an index, with
 * no replicated copy in memory.
 *
 * Mask (additive -inf, so masked probabilities are exactly 0):
 *   - causal != 0: key j is allowed for query row i iff j <= i (top-left
 *     alignment, the same as PyTorch SDPA's is_causal, also when Lq != Lk);
 *   - kv_len != NULL: key j is allowed iff j < clamp(kv_len[kv batch], 0, Lk);
 *     it masks keys only, every query row is computed;
 *   - the two combine by AND. A row with no allowed key is written as 0.
 * Keys are processed in tiles of 64. A masked key inside a tile that a row
 * reads still has its zero probability multiplied by its V row, so a
 * non-finite V value there (0 * Inf = NaN) reaches that row; tiles a row
 * does not read, and keys at or past kv_len, never do.
 *
 * Layout. Every tensor is contiguous row-major [batch, heads, seq, d], d
 * fastest (the PyTorch SDPA layout). q/k/v/o all have the element type
 * `dtype`: ATTN_BF16 (bfloat16; products accumulate in fp32 and the output is
 * rounded to nearest-even) or ATTN_F32. Base pointers must be 16-byte aligned.
 * All pointers are DEVICE pointers (HIP device memory of the current device).
 *
 * Ownership and concurrency. The caller owns every buffer. The library keeps
 * no state between calls and allocates nothing; calls are reentrant. Work is
 * enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 * call returns without synchronising: every input must be ready, and every
 * buffer the call writes must stay allocated and untouched, in that stream's
 * order. o must not alias q, k or v.
 *
 * Schedules. bf16 problems with d = 128 and Lk >= 4096 run an 8-wave
 * workgroup schedule, others a 4-wave one; both compute the same result to
 * within rounding. The environment variable ATTN_BF16_WAVES=4 or 8, read once
 * per process, forces one of them. Causal problems order their row blocks
 * longest-first across the K/V heads that share an XCD; ATTN_CHUNK_KV_MIB
 * (default 4, read once) bounds the K/V bytes of those heads.
 *
 * Errors. The return value is an attn_status. All argument checks run before
 * any HIP call. Device-resident values cannot be checked without a sync, so:
 * kv_len values are clamped to [0, Lk]; a cand2user value outside [0, B_u)
 * makes that candidate's output rows NaN.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = -1,       /* bad argument: NULL pointer, negative size, H % Hkv != 0,
                             misaligned pointer, non-finite or negative scale, size overflow,
                             bf16 with (Lk + 64) * d * 2 > 2^31 - 1 bytes per K/V head
                             (jagged: (max_Lk + 64) * Hkv * d * 2) */
  ATTN_EUNSUPPORTED = -2, /* head dim d not in {64, 128}, or unknown dtype */
  ATTN_ELAUNCH = -3,      /* the HIP launch reported an error. An error left pending by an
                             earlier HIP call on the calling thread is cleared before each
                             launch, so this status is about this call's launches only */
  ATTN_ESCRATCH = -4      /* attn_fwd_qknorm_noalloc: the normalised keys would not fit in
                             its fixed workspace (B * Hkv * Lk * d * 2 > 32 MiB) */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/*
 * Dense / causal / kv_len-masked / grouped-query attention forward.
 *   q      [B, H,   Lq, d]   queries
 *   k, v   [B, Hkv, Lk, d]   keys and values
 *   o      [B, H,   Lq, d]   output (written)
 *   kv_len [B] int32 or NULL (NULL: all Lk keys valid)
 *   scale  softmax scale; 0 means 1/sqrt(d); must be finite and >= 0
 * B, H, Lq, Lk >= 0 (an empty problem returns ATTN_OK and launches nothing;
 * Lk == 0 writes zeros), Hkv >= 1 with H % Hkv == 0.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o,
             int B, int H, int Hkv, int Lq, int Lk, int d,
             int causal, const int32_t* kv_len, float scale,
             int dtype, void* stream);

/*
 * In-kernel broadcast attention forward: candidate c attends over the K/V of
 * user cand2user[c], read in place (never replicated).
 *   q         [B_c, H,   Lq, d]  candidate queries
 *   k, v      [B_u, Hkv, Lk, d]  user keys and values
 *   o         [B_c, H,   Lq, d]  output (written)
 *   cand2user [B_c] int32, values in [0, B_u) (others give NaN rows)
 *   kv_len    [B_u] int32 or NULL, indexed by user
 * Other arguments as attn_fwd. The result is bit-identical to attn_fwd on
 * the replicated inputs k[cand2user], v[cand2user], kv_len[cand2user].
 */
int attn_fwd_bcast(const void* q, const void* k, const void* v, void* o,
                   const int32_t* cand2user, int B_c, int B_u,
                   int H, int Hkv, int Lq, int Lk, int d,
                   int causal, const int32_t* kv_len, float scale,
                   int dtype, void* stream);

/*
 * attn_fwd_bcast with the candidates packed in a given order. For short
 * query lengths the bf16 kernel packs several candidates into one workgroup,
 * which shares each K/V tile read among them ("How We Built TLX", Chinese
 * translation, "Case study 2: in-kernel broadcast optimisation for RecSys":
 * K/V read once per user); packed candidates of different users take one
 * pass each, with the other candidates' waves idle. Here workgroup slot s
 * holds candidate order[s], so an order that keeps each user's candidates
 * together (attn_bcast_group) restores one pass per workgroup for any
 * cand2user map.
 *   order [B_c] int32 in device memory: a permutation of 0 .. B_c-1 (not
 *         checked; a slot whose entry is out of range computes nothing, so an
 *         order that is not a permutation leaves rows unwritten)
 * Everything else as attn_fwd_bcast; the result is bit-identical to it (a
 * candidate's arithmetic does not depend on its slot). The fp32 path, which
 * does not pack candidates, ignores the order. Status codes as attn_fwd.
 */
int attn_fwd_bcast_grouped(const void* q, const void* k, const void* v, void* o,
                           const int32_t* cand2user, const int32_t* order, int B_c, int B_u,
                           int H, int Hkv, int Lq, int Lk, int d, int causal,
                           const int32_t* kv_len, float scale, int dtype, void* stream);

/*
 * Candidate grouping for attn_fwd_bcast_grouped: writes order[0 .. B_c-1], a
 * permutation of the candidates in which each user's candidates form one run
 * (users in increasing order; candidates whose user is out of [0, B_u) last,
 * and within a run in no fixed order). A counting sort in one workgroup,
 * enqueued on `stream`.
 *   cand2user [B_c] int32, device memory (read)
 *   order     [B_c] int32, device memory (written)
 *   work      [B_u + 1] int32, device memory: workspace, overwritten; it must
 *             not be in use by other work on the stream at the same time
 * Returns ATTN_OK (B_c = 0: nothing is enqueued), ATTN_EINVAL (B_c < 0,
 * B_u < 1 or B_u = INT_MAX, or a NULL pointer), ATTN_ELAUNCH.
 */
int attn_bcast_group(const int32_t* cand2user, int B_c, int B_u, int32_t* order, int32_t* work,
                     void* stream);

/*
 * Jagged (variable-length) attention forward: B sequences of different
 * lengths packed token by token, each attending over its own keys only.
 * The pages give this operation only as an article title ("Meta 造了个 Triton
 * 扩展 TLX..." page, link list, "Optimizing Jagged Flash Attention with
 * TLX"); the reading here is the plain one: offset arrays in place of B*L.
 *   q, o       [total_q,  H,   d]  total_q  = q_offsets[B]
 *   k, v       [total_kv, Hkv, d]  total_kv = kv_offsets[B]
 *   q_offsets  [B+1] int32, nondecreasing, q_offsets[0] = 0: sequence b owns
 *              query tokens q_offsets[b] .. q_offsets[b+1]-1
 *   kv_offsets [B+1] int32, the same for keys/values
 *   max_Lq, max_Lk  upper bounds of the lengths (the grid is sized on them);
 *              a longer sequence is cut: rows past max_Lq are not written,
 *              keys past max_Lk are ignored
 * Within a sequence the operation, masks (causal is top-left in local
 * indices) and element types are those of attn_fwd; a sequence with no keys
 * gives zero rows. Offsets live in device memory and are not checked
 * (lengths are clamped to [0, max]). bf16 needs (max_Lk + 64) * Hkv * d * 2
 * below 2^31 bytes. Other arguments and errors as attn_fwd.
 */
int attn_fwd_jagged(const void* q, const void* k, const void* v, void* o,
                    const int32_t* q_offsets, const int32_t* kv_offsets,
                    int B, int H, int Hkv, int max_Lq, int max_Lk, int d,
                    int causal, float scale, int dtype, void* stream);

/*
 * Fixed-block sparse attention forward: queries and keys are cut into blocks
 * of blk rows, and query block qb attends only to the key blocks kb with
 * block_mask[hm, qb, kb] != 0. The pages give this operation only as an
 * article title ("Meta 造了个 Triton 扩展 TLX..." page, link list, "TLX Block
 * Attention: ... Fixed-Block Sparse Self-Attention"); the reading here is the
 * plain one: a boolean block mask on top of the dense path's masks.
 *   q, k, v, o, B, H, Hkv, Lq, Lk, d, causal, kv_len, scale, dtype, stream
 *              as attn_fwd (dense layout)
 *   block_mask [mask_heads, ceil(Lq/blk), ceil(Lk/blk)] uint8 in device
 *              memory; nonzero = the block pair is attended
 *   mask_heads 1 (one mask for all heads and batch entries) or H (one per head)
 *   blk        block size, a positive multiple of 128 (a workgroup's query
 *              rows never straddle a block); ceil(Lk/blk) <= 1024
 * A key block left out is never loaded; rows whose blocks leave no valid key
 * are written as 0. Errors: ATTN_EINVAL also for a bad blk / mask_heads, a
 * NULL block_mask, or more than 1024 key blocks; otherwise as attn_fwd.
 */
int attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o,
                          const uint8_t* block_mask, int mask_heads, int blk,
                          int B, int H, int Hkv, int Lq, int Lk, int d,
                          int causal, const int32_t* kv_len, float scale,
                          int dtype, void* stream);

/*
 * Attention on RMS-normalised queries and keys (q-norm and k-norm fused with
 * the attention pass). The TLX pages ("How We Built TLX", Chinese translation,
 * the part on what compiler-inferred layouts make possible; link list, "...
 * Fusing Norms into GEMM and Attention via TLX") say normalisation can be
 * fused into attention kernels to save an intermediate memory round trip, and
 * name no norm; the reading here is RMS normalisation of every query and key
 * row over d, each with its own gain:
 *     q' = q / sqrt(mean(q^2) + eps) * gamma_q,  k' = k / sqrt(mean(k^2) + eps) * gamma_k
 * then attn_fwd(q', k', v). Queries are normalised in registers as the
 * attention kernel loads them (q' never reaches memory). Keys, which every
 * workgroup of their head reads many times, are normalised once by a
 * row-normalisation pass into k_norm, which the attention pass then reads.
 *   q, k, v, o, B, H, Hkv, Lq, Lk, d, causal, kv_len, scale, stream  as attn_fwd
 *   gamma_q, gamma_k  [d] fp32 device arrays, or NULL for ones
 *   eps               finite, >= 0
 *   k_norm            [B, Hkv, Lk, d] bf16 device workspace, written with the
 *                     normalised keys (rounded to nearest-even); the caller owns
 *                     it; it must not alias k
 * Only dtype = ATTN_BF16 (else ATTN_EUNSUPPORTED). q' and k' are rounded to
 * bf16 as MFMA operands. Two kernels are enqueued (keys, then attention).
 * Errors as attn_fwd, plus ATTN_EINVAL for a bad eps, a misaligned gain or
 * workspace, or a NULL / aliasing k_norm when there are keys.
 */
int attn_fwd_qknorm(const void* q, const void* k, const void* v, void* o,
                    const float* gamma_q, const float* gamma_k, float eps, void* k_norm,
                    int B, int H, int Hkv, int Lq, int Lk, int d,
                    int causal, const int32_t* kv_len, float scale, int dtype, void* stream);

/*
 * attn_fwd_qknorm without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The same arguments, results and checks
 * as attn_fwd_qknorm, minus k_norm: the normalised keys go to a 32 MiB array
 * the library defines in device memory, one per GPU, held from the first use
 * on that GPU until the process ends. The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); its first call on a
 * device looks the array up with hipGetSymbolAddress (ATTN_ELAUNCH if that
 * fails).
 * Limit: B * Hkv * Lk * d * 2 <= 32 MiB (the GQA workload B=1, Hkv=8,
 * Lk=16384, d=128 fits exactly); larger problems return ATTN_ESCRATCH after
 * every other check and before any HIP call.
 * Concurrency: all calls on one GPU share that array. Calls whose work can
 * overlap on one GPU (two host threads, or two streams not ordered against
 * each other) race on it and give wrong results: serialise them, e.g. on one
 * stream. Every call writes the keys it reads first, so nothing needs
 * clearing between calls.
 */
int attn_fwd_qknorm_noalloc(const void* q, const void* k, const void* v, void* o,
                            const float* gamma_q, const float* gamma_k, float eps,
                            int B, int H, int Hkv, int Lq, int Lk, int d,
                            int causal, const int32_t* kv_len, float scale, int dtype,
                            void* stream);

/*
 * In-kernel broadcast linear layer: one linear layer over the concatenated
 * features [x_user[cand2user[c]], x_cand[c]] of every candidate c, computed
 * without replicating the user features. "How We Built TLX" (Chinese
 * translation, "Case study 2: in-kernel broadcast optimisation for RecSys")
 * names this linear-compression kernel and the three steps that sped it up
 * (splitting the matrix product, aligning memory, fusing the broadcast) but
 * gives no formula; the reading here is the plain one:
 *     y[c] = x_cand[c] w_cand^T + z[cand2user[c]],
 *     z[u] = x_user[u] w_user^T + bias            (once per user)
 * with w = [w_user | w_cand] split by columns.
 *   x_user    [B_u, K_u] bf16         user features
 *   x_cand    [B_c, K_c] bf16         candidate features
 *   w         [N, K_u + K_c] bf16     weight, user columns first (the
 *                                     nn.Linear layout: one row per output)
 *   bias      [N] fp32 or NULL
 *   cand2user [B_c] int32, values in [0, B_u) (others give NaN rows)
 *   y         [B_c, N] of y_dtype (ATTN_BF16: rounded to nearest-even from
 *             the fp32 sum; ATTN_F32), written
 *   z         [B_u, N] fp32, written with the user half plus the bias; the
 *             caller owns it (it is also a result) and it must not alias y
 * Products are exact in fp32 and accumulate in fp32. All pointers are device
 * pointers, 16-byte aligned. K_u and K_c are multiples of 8, N a multiple of
 * 4, K_u + K_c <= 2^20, N * (K_u + K_c) * 2 < 2^31 and, when y is bf16 and
 * B_c > 0, N < 2^22; either K may be 0 (that half contributes nothing).
 * B_c > 0 needs B_u >= 1. Two kernels are enqueued on `stream` (z, then y);
 * the call does not synchronise. Errors: ATTN_EINVAL for a bad size, a NULL
 * or misaligned pointer that the sizes make used; ATTN_EUNSUPPORTED for
 * another y_dtype; ATTN_ELAUNCH.
 */
int ikbo_linear(const void* x_user, const void* x_cand, const void* w, const float* bias,
                const int32_t* cand2user, void* y, float* z,
                int B_u, int B_c, int K_u, int K_c, int N, int y_dtype, void* stream);

/* Static, human-readable text for a status code (never NULL). */
const char* attn_strerror(int status);

/* ABI version: major * 100 + minor (101: attn_fwd_jagged; 102: attn_fwd_block_sparse;
 * 103: ikbo_linear; 104: attn_fwd_qknorm; 105: attn_fwd_qknorm_noalloc;
 * 106: attn_fwd_bcast_grouped, attn_bcast_group). */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
