// fp32 tiled attention forward (fp32 in, fp32 out, fp32 arithmetic).
//
// Same operation and online softmax as the bf16 kernel (tutorial page "Guide
// de programmation pour la programmation GPU par tuiles de NVIDIA : de cuTile
// et des noyaux Triton a Flash Attention", flash-attention paragraph), kept in
// fp32 end to end so the result stays within 1e-4 of the exact value. This
// path serves small fp32 problems: four lanes per query row, each holding a
// quarter of the row's columns (the score's partial dot products are summed
// across the four lanes with two DPP adds), K/V tiles of 32 keys staged in
// LDS, VALU FMAs for both products. It handles the dense, broadcast, jagged
// and block-sparse layouts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_params.h"

namespace attn {

constexpr int kF32Rows = 64;   // query rows per workgroup
constexpr int kF32Split = 4;   // lanes per query row (consecutive lanes of a DPP quad)
constexpr int kF32Keys = 32;   // keys per LDS tile

// Sum over the four lanes of a quad. Both steps add the same two values in
// either order, so all four lanes get the same bits.
__device__ __forceinline__ float quad_sum(float x) {
  // quad_perm [1,0,3,2], then [2,3,0,1]
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  return x;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF32Rows * kF32Split) void attn_fwd_f32_kernel(const Params p) {
  constexpr int DL = D / kF32Split;   // columns per lane
  constexpr int kThreads = kF32Rows * kF32Split;
  __shared__ float ks[kF32Keys][D];
  __shared__ float vs[kF32Keys][D];
  const int tid = threadIdx.x;
  const int c0 = (tid % kF32Split) * DL;   // this lane's columns c0 .. c0 + DL - 1
  const int nrb = (p.Lq + kF32Rows - 1) / kF32Rows;
  const int mt = blockIdx.x % nrb;
  const int bh = blockIdx.x / nrb;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int g = h / (p.H / p.Hkv);
  const int row = mt * kF32Rows + tid / kF32Split;
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
    if (kvb < 0 || kvb >= p.NKV) {  // out-of-range user: NaN rows
      if (row_ok)
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

  float q[DL], o[DL];
  for (int d = 0; d < DL; ++d) {
    q[d] = row_ok ? qg[qoff + d] : 0.f;
    o[d] = 0.f;
  }
  const size_t kvbase = jagged ? (size_t)p.kv_offsets[b] * kv_rs + (size_t)g * D
                               : ((size_t)kvb * p.Hkv + g) * p.Lk * D;
  const float* __restrict__ kg = (const float*)p.k + kvbase;
  const float* __restrict__ vg = (const float*)p.v + kvbase;
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.c;

  // block-sparse: the workgroup's 64 rows lie in one query block (blk is a
  // multiple of 128); skip the key tiles of blocks its mask row leaves out
  const uint8_t* mrow = nullptr;
  if (p.block_mask != nullptr) {
    const int qblk = min(mt * kF32Rows / p.blk, p.nQB - 1);
    mrow = p.block_mask + ((size_t)(p.mask_heads == 1 ? 0 : h) * p.nQB + qblk) * p.nKB;
  }
  for (int t = 0; t < ntiles; ++t) {
    if (mrow != nullptr && mrow[(t * kF32Keys) / p.blk] == 0) continue;   // uniform
    __syncthreads();
    for (int e = tid; e < kF32Keys * D; e += kThreads) {
      const int j = e / D, d = e % D;
      const int key = t * kF32Keys + j;
      ks[j][d] = key < kread ? kg[(size_t)key * kv_rs + d] : 0.f;
      vs[j][d] = key < kread ? vg[(size_t)key * kv_rs + d] : 0.f;
    }
    __syncthreads();
    float s[kF32Keys];
    float mx = -INFINITY;
    for (int j = 0; j < kF32Keys; ++j) {
      // two partial sums over this lane's columns, then the quad's sum
      float a0 = 0.f, a1 = 0.f;
      for (int d = 0; d < DL; d += 2) {
        a0 = __builtin_fmaf(q[d], ks[j][c0 + d], a0);
        a1 = __builtin_fmaf(q[d + 1], ks[j][c0 + d + 1], a1);
      }
      const float acc = quad_sum(a0 + a1);
      const int key = t * kF32Keys + j;
      bool dead = key >= nvalid;
      if (CAUSAL) dead = dead || key > row;
      s[j] = dead ? -INFINITY : acc * c;  // base-2 logits
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
    for (int d = 0; d < DL; ++d) o[d] *= alpha;
    for (int j = 0; j < kF32Keys; ++j) {
      const float pj = exp2f(s[j] - m_use);
      l_run += pj;
      for (int d = 0; d < DL; ++d) o[d] = __builtin_fmaf(pj, vs[j][c0 + d], o[d]);
    }
  }
  if (row_ok) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    for (int d = 0; d < DL; ++d) og[qoff + d] = o[d] * inv;
  }
}

hipError_t launch_f32(const Params& p, int D, bool causal, hipStream_t stream) {
  // An error left pending by an earlier HIP call on this thread is dropped
  // here, so that the status returned after the launch is this launch's.
  (void)hipGetLastError();
  const int nrb = (p.Lq + kF32Rows - 1) / kF32Rows;
  dim3 grid((unsigned)((size_t)p.NB * p.H * nrb)), block(kF32Rows * kF32Split);
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
