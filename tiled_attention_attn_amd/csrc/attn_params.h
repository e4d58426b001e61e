// Launch parameters shared by the host dispatcher and the attention kernels.
#pragma once
#include <stdint.h>

namespace attn {

// One attention problem as the kernels see it. Dense problems have
// cand2user == nullptr and NKV == NB; the broadcast problem indexes the K/V
// batch of query batch entry b as cand2user[b]. Jagged problems (q_offsets
// != nullptr) pack the sequences of a batch token by token: Q/O are
// [total_q, H, D] and K/V [total_kv, Hkv, D]; sequence b holds rows
// q_offsets[b] .. q_offsets[b+1]-1 (K/V likewise), and Lq / Lk are the
// largest lengths (the grid is sized on them).
struct Params {
  const void* q;             // [NB, H, Lq, D]    (jagged: [total_q, H, D])
  const void* k;             // [NKV, Hkv, Lk, D] (jagged: [total_kv, Hkv, D])
  const void* v;             // [NKV, Hkv, Lk, D] (jagged: [total_kv, Hkv, D])
  void* o;                   // [NB, H, Lq, D]    (jagged: [total_q, H, D])
  const int32_t* kv_len;     // [NKV] or nullptr
  const int32_t* cand2user;  // [NB] or nullptr
  const int32_t* cand_order; // [NB] or nullptr: the candidate each packed slot holds (broadcast)
  const int32_t* q_offsets;  // [NB + 1] or nullptr (dense layout)
  const int32_t* kv_offsets; // [NB + 1], set iff q_offsets is
  const uint8_t* block_mask; // [mask_heads, nQB, nKB] or nullptr (no block sparsity)
  int blk, nQB, nKB, mask_heads;  // block size (keys = queries), mask extents
  int NB, NKV, H, Hkv, Lq, Lk;
  float c;                   // scale * log2(e): softmax runs in base 2
  // Work decomposition (filled by the host dispatcher).
  int P;      // 32-row query blocks per (batch entry, head), padded so tiles never straddle
  int G;      // batch entries packed into one workgroup (P < 4 only)
  int nMT;    // workgroups per (batch group, head)
  int NG;     // batch groups = ceil(NB / G)
  int T;      // total workgroups
  int chunk;  // logical tiles kept together on one XCD (0 = no remap)
  int units;  // dense: (batch group, K/V head) units per chunk; causal tiles of a
              // chunk run row block by row block across its units (heaviest first)
  int waves;  // waves per workgroup of the bf16 kernel (4 or 8)
  // Query RMS normalisation at load time (bf16 kernel): each query row x
  // becomes x / sqrt(mean(x^2) + eps) * gamma_q (gamma_q may be nullptr: ones).
  int qnorm;
  float eps;
  const float* gamma_q;      // [D] or nullptr
};

}  // namespace attn
