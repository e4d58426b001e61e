// bf16 fused tiled attention forward for gfx950 (CDNA4): bf16 MFMA with fp32
// accumulation, online softmax in registers, K/V double-buffered in LDS.
//
// Method: the tutorial page "Guide de programmation pour la programmation GPU
// par tuiles de NVIDIA : de cuTile et des noyaux Triton a Flash Attention"
// (flash-attention paragraph, conclusion): attention over key tiles with a
// running row max and row sum, so the score matrix never leaves registers.
// Broadcast: "How We Built TLX" (Chinese translation, "Case study 2: in-kernel
// broadcast optimisation for RecSys"): K/V reads are shared by candidates of
// the same user and indexed in-kernel instead of being replicated.
//
// Work decomposition. A workgroup is 4 waves; each wave owns 32 query rows of
// one (batch entry, head). The wave computes the transposed score tile
//     S^T[key, query] = K_tile . Q^T      (v_mfma_f32_32x32x16_bf16)
// so that in the MFMA accumulator layout each lane holds ONE query (column
// lane%32) and 16 keys per 32-key block: the row max and row sum are in-lane
// plus one exchange between the two lane halves. The probabilities stay in
// that layout and feed the second product directly as the B operand:
//     O^T[d, query] += V^T . P^T          (v_mfma_f32_32x32x16_bf16)
// whose accumulator again has one query per lane, so the online-softmax
// rescale by alpha is lane-local. V^T operands come from row-major V in LDS
// through the gfx950 transposing LDS read (ds_read_b64_tr_b16).
//
// MFMA 32x32x16 bf16 lane layout (checked on the device):
//   A (32 x 16): lane l holds row l%32, k-slots (l/32)*8 .. +7
//   B (16 x 32): lane l holds col l%32, k-slots (l/32)*8 .. +7
//   C (32 x 32): lane l holds col l%32, rows (i/4)*8 + (l/32)*4 + i%4, i < 16
// The k-slot -> key assignment of the PV product is free as long as A and B
// agree; it is chosen to match the C layout of S^T, so P needs no shuffle:
//   slot j of half h in PV step t  <->  key 16t + (j/4)*8 + 4h + j%4.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_params.h"

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;

template <int D>
struct Tile {
  static constexpr int BN = (D == 128) ? 64 : 128;  // keys per tile
  static constexpr int NC = D / 8;                   // 16-byte chunks per K/V row
  static constexpr int KB = BN / 32;                 // 32-key blocks per tile
  static constexpr int DB = D / 32;                  // 32-wide d blocks of O^T
  static constexpr int QS = D / 16;                  // k-steps of the QK^T product
  static constexpr int PS = BN / 16;                 // k-steps of the PV product
  static constexpr int CHUNKS = BN * NC;             // 16-byte chunks per K (or V) tile
  static constexpr int LOADS = CHUNKS / kThreads;    // 16-byte loads per thread per matrix
  static_assert(CHUNKS % kThreads == 0, "tile must split evenly over the workgroup");
};

// LDS swizzles (16-byte chunk granularity, bijective within a row).
// K rows are read 16 bytes per lane with consecutive lanes on consecutive
// rows: XOR with the row index spreads them over all banks.
template <int NC>
__device__ __forceinline__ int k_swz(int row, int c) { return c ^ (row & (NC - 1)); }
// V rows are read by the transposing load: a 16-lane group touches 4
// consecutive rows x 32 bytes; XOR of the 32-byte pair index with row%4
// keeps those 4 pairs in distinct banks.
__device__ __forceinline__ int v_swz(int row, int c) { return c ^ ((row & 3) << 1); }

__device__ __forceinline__ float wave_max_halves(float x) {
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float wave_sum_halves(float x) {
  return x + __shfl_xor(x, 32, 64);
}

// Map the hardware workgroup id to a logical tile so that runs of `chunk`
// consecutive logical tiles (which share K/V) land on one XCD. Workgroups
// are dispatched round-robin over the 8 XCDs, so XCD x runs ids x, x+8, ...
__device__ __forceinline__ int xcd_remap(int w, int T, int chunk) {
  constexpr int NX = 8;
  if (chunk <= 0) return w;
  int full = (T / (NX * chunk)) * NX * chunk;
  if (w >= full) return w;
  int x = w % NX, s = w / NX;
  return ((s / chunk) * NX + x) * chunk + (s % chunk);
}

struct WaveTask {
  int batch;   // query-side batch entry
  int row0;    // first query row of the wave
  int kvb;     // K/V batch entry (user for the broadcast variant)
  bool valid;  // rows exist
  bool bad;    // kvb out of range: output NaN
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(const Params p) {
  using TL = Tile<D>;
  constexpr int BN = TL::BN, NC = TL::NC, KB = TL::KB, DB = TL::DB, QS = TL::QS, PS = TL::PS;
  constexpr int LOADS = TL::LOADS;

  __shared__ u32x4 smem[2][2][TL::CHUNKS];  // [buffer][K=0, V=1][chunk]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;   // which k-slot half of the MFMA operands
  const int col = lane & 31;    // the query this lane owns

  // ---- decode the logical tile --------------------------------------------
  const int L = xcd_remap(blockIdx.x, p.T, p.chunk);
  const int HPG = p.H / p.Hkv;
  int bgrp, h, mt;
  if (p.cand2user == nullptr) {
    // dense: ((b * Hkv + g) * nMT + mt') * HPG + hq; causal runs heavy tiles first
    int hq = L % HPG;
    int r = L / HPG;
    int mtr = r % p.nMT;
    r /= p.nMT;
    int g = r % p.Hkv;
    bgrp = r / p.Hkv;
    h = g * HPG + hq;
    mt = CAUSAL ? (p.nMT - 1 - mtr) : mtr;
  } else {
    // broadcast: ((g * HPG + hq) * NG + bgrp) * nMT + mt': neighbouring tiles
    // are neighbouring candidates of one head, which usually share a user.
    int mtr = L % p.nMT;
    int r = L / p.nMT;
    bgrp = r % p.NG;
    r /= p.NG;
    h = r;  // g * HPG + hq
    mt = CAUSAL ? (p.nMT - 1 - mtr) : mtr;
  }
  const int g = h / HPG;

  // Every thread can derive the task of any wave (needed for shared loop bounds).
  auto task_of = [&](int w) -> WaveTask {
    WaveTask t;
    if (p.G == 1) {
      t.batch = bgrp;
      t.row0 = (mt * kWaves + w) * kRowsPerWave;
    } else {
      t.batch = bgrp * p.G + w / p.P;
      t.row0 = (w % p.P) * kRowsPerWave;
    }
    t.valid = t.batch < p.NB && t.row0 < p.Lq;
    t.kvb = t.batch;
    t.bad = false;
    if (t.valid && p.cand2user != nullptr) {
      t.kvb = p.cand2user[t.batch];
      t.bad = (t.kvb < 0) || (t.kvb >= p.NKV);
    }
    return t;
  };

  const WaveTask me = task_of(wave);
  const size_t q_head = ((size_t)me.batch * p.H + h) * (size_t)p.Lq;  // row index base
  const __bf16* __restrict__ qg = (const __bf16*)p.q;
  __bf16* __restrict__ og = (__bf16*)p.o;

  // Candidates with an out-of-range user index get NaN rows.
  if (me.valid && me.bad) {
    const int row = me.row0 + col;
    if (row < p.Lq) {
      __bf16* orow = og + (q_head + row) * D;
      const __bf16 nanv = __builtin_bit_cast(__bf16, (unsigned short)0x7FC0);
      for (int d = half * (D / 2); d < (half + 1) * (D / 2); ++d) orow[d] = nanv;
    }
  }

  const float c = p.c;

  // One pass per distinct K/V batch among the waves (normally exactly one).
  for (int lead = 0; lead < kWaves; ++lead) {
    const WaveTask lt = task_of(lead);
    if (!lt.valid || lt.bad) continue;
    bool seen = false;
    for (int w = 0; w < lead; ++w) {
      const WaveTask tw = task_of(w);
      if (tw.valid && !tw.bad && tw.kvb == lt.kvb) seen = true;
    }
    if (seen) continue;
    const int kvb = lt.kvb;

    int nvalid = p.Lk;
    if (p.kv_len != nullptr) nvalid = min(max(p.kv_len[kvb], 0), p.Lk);

    // keys needed by a wave: causal rows r allow keys <= r
    auto keys_needed = [&](const WaveTask& t) -> int {
      int n = nvalid;
      if (CAUSAL) n = min(n, min(t.row0 + kRowsPerWave, p.Lq));
      return n;
    };
    int ntiles = 0;
    for (int w = 0; w < kWaves; ++w) {
      const WaveTask t = task_of(w);
      if (t.valid && !t.bad && t.kvb == kvb) ntiles = max(ntiles, (keys_needed(t) + BN - 1) / BN);
    }
    const bool active = me.valid && !me.bad && me.kvb == kvb;
    const int my_keys = active ? keys_needed(me) : 0;
    const int my_tiles = (my_keys + BN - 1) / BN;

    const size_t kv_head = ((size_t)kvb * p.Hkv + g) * (size_t)p.Lk;
    const __bf16* __restrict__ kg = (const __bf16*)p.k + kv_head * D;
    const __bf16* __restrict__ vg = (const __bf16*)p.v + kv_head * D;

    // Q^T operand: lane holds query row0+col, d = 16*s + 8*half + 0..7.
    bf16x8 qreg[QS];
    {
      const int row = me.row0 + col;
      const bool ok = active && row < p.Lq;
      const __bf16* qrow = qg + (q_head + (ok ? row : 0)) * D;
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (ok) x = *(const u32x4*)(qrow + 16 * s + 8 * half);
        qreg[s] = __builtin_bit_cast(bf16x8, x);
      }
    }

    f32x16 oacc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[b][i] = 0.f;
    float m_run = -INFINITY;  // running max of raw scores (this lane's query)
    float l_run = 0.f;        // running sum over this lane's keys only

    // global -> register staging of one K and one V tile
    u32x4 kst[LOADS], vst[LOADS];
    auto load_tile = [&](int t) {
#pragma unroll
      for (int n = 0; n < LOADS; ++n) {
        const int e = tid + n * kThreads;
        const int row = e / NC, cc = e % NC;
        const int key = t * BN + row;
        u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
        if (key < p.Lk) {
          zk = *(const u32x4*)(kg + (size_t)key * D + cc * 8);
          zv = *(const u32x4*)(vg + (size_t)key * D + cc * 8);
        }
        kst[n] = zk;
        vst[n] = zv;
      }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
      for (int n = 0; n < LOADS; ++n) {
        const int e = tid + n * kThreads;
        const int row = e / NC, cc = e % NC;
        smem[buf][0][row * NC + k_swz<NC>(row, cc)] = kst[n];
        smem[buf][1][row * NC + v_swz(row, cc)] = vst[n];
      }
    };

    auto compute_tile = [&](int t, int buf) {
      // ---- S^T = K . Q^T -------------------------------------------------
      f32x16 sacc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
      for (int s = 0; s < QS; ++s) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int row = kb * 32 + col;
          const int cc = 2 * s + half;
          const bf16x8 a = __builtin_bit_cast(bf16x8, smem[buf][0][row * NC + k_swz<NC>(row, cc)]);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc[kb], 0, 0, 0);
        }
      }
      // ---- mask (boundary tiles only) ---------------------------------------
      const int key0 = t * BN;
      const int qrow = me.row0 + col;
      const bool need_mask = (key0 + BN > nvalid) || (CAUSAL && key0 + BN - 1 > me.row0);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
            bool dead = key >= nvalid;
            if (CAUSAL) dead = dead || key > qrow;
            if (dead) sacc[kb][i] = -INFINITY;
          }
      }
      // ---- online softmax (base 2, scale folded into c) --------------------
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = wave_max_halves(mx);
      const float m_new = fmaxf(m_run, mx);
      const float mc = (m_new == -INFINITY) ? 0.f : m_new * c;
      const float alpha = __builtin_amdgcn_exp2f(m_run * c - mc);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], c, -mc));
          sacc[kb][i] = pv;
          rs += pv;
        }
      l_run = l_run * alpha + rs;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[b][i] *= alpha;
      }
      // ---- O^T += V^T . P^T --------------------------------------------------
      const int il = lane & 15;
      const int grp = lane >> 4;  // 16-lane group: d half = grp & 1, k half = grp >> 1
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
        bf16x8 pb;
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[j] = (__bf16)sacc[ps >> 1][(ps & 1) * 8 + j];
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          // transposing read: source role il addresses V[row][dcol .. dcol+3];
          // result lane il gets V[key0 + s][dbase + il] for s = 0..3.
          const int dcol = b * 32 + (grp & 1) * 16 + 4 * (il & 3);
          const int cc = dcol >> 3, within = (dcol & 7) * 2;
          const int r1 = ps * 16 + half * 4 + (il >> 2);
          const int r2 = r1 + 8;
          const LDS_AS char* vb = (const LDS_AS char*)&smem[buf][1][0];
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (LDS_AS bf16x4*)(vb + (r1 * NC + v_swz(r1, cc)) * 16 + within));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (LDS_AS bf16x4*)(vb + (r2 * NC + v_swz(r2, cc)) * 16 + within));
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[b], 0, 0, 0);
        }
      }
    };

    if (ntiles > 0) {
      load_tile(0);
      store_tile(0);
      __syncthreads();
      for (int t = 0; t < ntiles; ++t) {
        const bool more = t + 1 < ntiles;
        if (more) load_tile(t + 1);
        if (t < my_tiles) compute_tile(t, t & 1);
        if (more) store_tile((t + 1) & 1);
        __syncthreads();
      }
    }

    // ---- epilogue: O = O^T / l, round to bf16, store ---------------------------
    if (active) {
      const float l = wave_sum_halves(l_run);
      const float inv = (l > 0.f) ? 1.f / l : 0.f;
      const int row = me.row0 + col;
      if (row < p.Lq) {
        __bf16* orow = og + (q_head + row) * D;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int m4 = 0; m4 < 4; ++m4) {
            bf16x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = (__bf16)(oacc[b][m4 * 4 + j] * inv);
            *(bf16x4*)(orow + b * 32 + m4 * 8 + half * 4) = w;
          }
      }
    }
  }
}

// Host-side launchers (one per template instance).
hipError_t launch_bf16(const Params& p, int D, bool causal, hipStream_t stream) {
  dim3 grid(p.T), block(kThreads);
  if (D == 128) {
    if (causal) hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, false>), grid, block, 0, stream, p);
  } else {
    if (causal) hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

int bf16_rows_per_workgroup() { return kWaves * kRowsPerWave; }

}  // namespace attn
