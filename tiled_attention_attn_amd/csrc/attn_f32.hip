// fp32 tiled attention forward (fp32 in, fp32 out, fp32 arithmetic).
//
// Same operation and online softmax as the bf16 kernel (tutorial page "Guide
// de programmation pour la programmation GPU par tuiles de NVIDIA : de cuTile
// et des noyaux Triton a Flash Attention", flash-attention paragraph), kept in
// fp32 end to end so the result stays within 1e-4 of the exact value. This
// path serves small fp32 problems, where the run time is the serial work of
// one row, so a workgroup spreads each row over 16 lanes: four lanes hold a
// quarter of the row's columns each (a score is the quad's sum of four
// partial dot products, two DPP adds), and four key groups of 256 threads take
// every fourth 16-key tile, each with its own online-softmax state; at the
// end the groups' states are merged through LDS (the same rescaling as one
// online-softmax step). K/V tiles are staged in LDS, both products are VALU
// FMAs. It handles the dense, broadcast, jagged and block-sparse layouts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_params.h"

namespace attn {

constexpr int kF32Rows = 64;   // query rows per workgroup
constexpr int kF32Split = 4;   // lanes per query row (consecutive lanes of a DPP quad)
constexpr int kF32Groups = 4;  // key groups per workgroup (each takes every fourth tile)
constexpr int kF32Keys = 16;   // keys per LDS tile

// Sum over the four lanes of a quad. Both steps add the same two values in
// either order, so all four lanes get the same bits.
__device__ __forceinline__ float quad_sum(float x) {
  // quad_perm [1,0,3,2], then [2,3,0,1]
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  return x;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF32Rows * kF32Split * kF32Groups) void attn_fwd_f32_kernel(const Params p) {
  constexpr int DL = D / kF32Split;                   // columns per lane
  constexpr int kGroupThreads = kF32Rows * kF32Split;
  constexpr int kTile = kF32Keys * D;                 // floats of one K (or V) tile
  constexpr int kMergeRow = D + 2;                    // o, m, l of one row in the merge area
  constexpr int kTiles = 2 * kF32Groups * kTile;
  constexpr int kMerge = (kF32Groups - 1) * kF32Rows * kMergeRow;
  // the groups' K/V tiles during the loop, the groups' states at the end
  __shared__ float lds[kTiles > kMerge ? kTiles : kMerge];
  const int tid = threadIdx.x;
  const int kg = tid / kGroupThreads;                 // key group
  const int gt = tid % kGroupThreads;                 // thread within the group
  const int c0 = (gt % kF32Split) * DL;               // this lane's columns c0 .. c0 + DL - 1
  const int rl = gt / kF32Split;                      // row within the workgroup
  float* ks = lds + (2 * kg) * kTile;                 // [kF32Keys][D] of this group
  float* vs = lds + (2 * kg + 1) * kTile;
  const int nrb = (p.Lq + kF32Rows - 1) / kF32Rows;
  const int mt = blockIdx.x % nrb;
  const int bh = blockIdx.x / nrb;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int g = h / (p.H / p.Hkv);
  const int row = mt * kF32Rows + rl;
  // Dense rows of one (batch, head) are D elements apart; jagged tokens are
  // packed [total, heads, D] with sequence b starting at offsets[b].
  const bool jagged = p.q_offsets != nullptr;
  const int q_rs = jagged ? p.H * D : D;
  const int kv_rs = jagged ? p.Hkv * D : D;
  const int lq = jagged ? min(max(p.q_offsets[b + 1] - p.q_offsets[b], 0), p.Lq) : p.Lq;
  const bool row_ok = row < lq;

  const float* __restrict__ qg = (const float*)p.q;
  float* __restrict__ og = (float*)p.o;
  const size_t qbase = jagged ? (size_t)p.q_offsets[b] * q_rs + (size_t)h * D
                              : ((size_t)b * p.H + h) * p.Lq * D;
  const size_t qoff = qbase + (size_t)(row_ok ? row : 0) * q_rs + c0;

  int kvb = b;
  if (p.cand2user != nullptr) {
    kvb = p.cand2user[b];
    if (kvb < 0 || kvb >= p.NKV) {  // out-of-range user: NaN rows (the whole workgroup returns)
      if (row_ok && kg == 0)
        for (int d = 0; d < DL; ++d) og[qoff + d] = __builtin_nanf("");
      return;
    }
  }
  int nvalid = jagged ? min(max(p.kv_offsets[b + 1] - p.kv_offsets[b], 0), p.Lk) : p.Lk;
  if (p.kv_len != nullptr) nvalid = min(max(p.kv_len[kvb], 0), p.Lk);
  // keys that may be read: a jagged sequence must not read its neighbours;
  // keys past the valid ones are masked; they are not read either (zero K and
  // V), so that uninitialised padding past kv_len cannot reach the output
  // through 0 * NaN
  const int kread = nvalid;
  int nkeys = nvalid;
  if (CAUSAL) nkeys = min(nkeys, min(mt * kF32Rows + kF32Rows, lq));
  const int ntiles = (nkeys + kF32Keys - 1) / kF32Keys;
  const int rounds = (ntiles + kF32Groups - 1) / kF32Groups;   // the same for every group

  float q[DL], o[DL];
  for (int d = 0; d < DL; ++d) {
    q[d] = row_ok ? qg[qoff + d] : 0.f;
    o[d] = 0.f;
  }
  const size_t kvbase = jagged ? (size_t)p.kv_offsets[b] * kv_rs + (size_t)g * D
                               : ((size_t)kvb * p.Hkv + g) * p.Lk * D;
  const float* __restrict__ kgp = (const float*)p.k + kvbase;
  const float* __restrict__ vgp = (const float*)p.v + kvbase;
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.c;

  // block-sparse: the workgroup's 64 rows lie in one query block (blk is a
  // multiple of 128); the key tiles of blocks its mask row leaves out are skipped
  const uint8_t* mrow = nullptr;
  if (p.block_mask != nullptr) {
    const int qblk = min(mt * kF32Rows / p.blk, p.nQB - 1);
    mrow = p.block_mask + ((size_t)(p.mask_heads == 1 ? 0 : h) * p.nQB + qblk) * p.nKB;
  }
  // Every group runs the same rounds (so every barrier is reached by every
  // thread); a group whose tile is past the end or masked out only waits.
  for (int r = 0; r < rounds; ++r) {
    const int t = r * kF32Groups + kg;
    const bool live = t < ntiles && (mrow == nullptr || mrow[(t * kF32Keys) / p.blk] != 0);
    __syncthreads();
    if (live) {
      for (int e = gt; e < kTile; e += kGroupThreads) {
        const int j = e / D, d = e % D;
        const int key = t * kF32Keys + j;
        ks[e] = key < kread ? kgp[(size_t)key * kv_rs + d] : 0.f;
        vs[e] = key < kread ? vgp[(size_t)key * kv_rs + d] : 0.f;
      }
    }
    __syncthreads();
    if (!live) continue;
    float sc[kF32Keys];
    float mx = -INFINITY;
    for (int j = 0; j < kF32Keys; ++j) {
      // two partial sums over this lane's columns, then the quad's sum
      float a0 = 0.f, a1 = 0.f;
      for (int d = 0; d < DL; d += 2) {
        a0 = __builtin_fmaf(q[d], ks[j * D + c0 + d], a0);
        a1 = __builtin_fmaf(q[d + 1], ks[j * D + c0 + d + 1], a1);
      }
      const float acc = quad_sum(a0 + a1);
      const int key = t * kF32Keys + j;
      bool dead = key >= nvalid;
      if (CAUSAL) dead = dead || key > row;
      sc[j] = dead ? -INFINITY : acc * c;  // base-2 logits
      mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
    for (int d = 0; d < DL; ++d) o[d] *= alpha;
    for (int j = 0; j < kF32Keys; ++j) {
      const float pj = exp2f(sc[j] - m_use);
      l_run += pj;
      for (int d = 0; d < DL; ++d) o[d] = __builtin_fmaf(pj, vs[j * D + c0 + d], o[d]);
    }
  }
  // Merge: groups 1.. store their row states, group 0 rescales all of them to
  // the largest reference (a group that saw no key of a row has m = -inf and
  // weighs nothing) and writes the row.
  __syncthreads();
  if (kg > 0) {
    float* st = lds + ((kg - 1) * kF32Rows + rl) * kMergeRow;
    for (int d = 0; d < DL; ++d) st[c0 + d] = o[d];
    if (c0 == 0) {
      st[D] = m_run;
      st[D + 1] = l_run;
    }
  }
  __syncthreads();
  if (kg == 0 && row_ok) {
    float m = m_run;
    for (int k = 1; k < kF32Groups; ++k) m = fmaxf(m, lds[((k - 1) * kF32Rows + rl) * kMergeRow + D]);
    const float m_use = (m == -INFINITY) ? 0.f : m;
    const float f0 = exp2f(m_run - m_use);
    float l = l_run * f0;
    for (int d = 0; d < DL; ++d) o[d] *= f0;
    for (int k = 1; k < kF32Groups; ++k) {
      const float* st = lds + ((k - 1) * kF32Rows + rl) * kMergeRow;
      const float f = exp2f(st[D] - m_use);
      l = __builtin_fmaf(st[D + 1], f, l);
      for (int d = 0; d < DL; ++d) o[d] = __builtin_fmaf(st[c0 + d], f, o[d]);
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    for (int d = 0; d < DL; ++d) og[qoff + d] = o[d] * inv;
  }
}

hipError_t launch_f32(const Params& p, int D, bool causal, hipStream_t stream) {
  // An error left pending by an earlier HIP call on this thread is dropped
  // here, so that the status returned after the launch is this launch's.
  (void)hipGetLastError();
  const int nrb = (p.Lq + kF32Rows - 1) / kF32Rows;
  dim3 grid((unsigned)((size_t)p.NB * p.H * nrb)), block(kF32Rows * kF32Split * kF32Groups);
  if (D == 128) {
    if (causal) hipLaunchKernelGGL((attn_fwd_f32_kernel<128, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((attn_fwd_f32_kernel<128, false>), grid, block, 0, stream, p);
  } else {
    if (causal) hipLaunchKernelGGL((attn_fwd_f32_kernel<64, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((attn_fwd_f32_kernel<64, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace attn
