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
// Work decomposition. A workgroup is 4 waves, one per SIMD; each wave owns 64
// query rows of one (batch entry, head) as two 32-query blocks, so every K or
// V operand read from LDS feeds two MFMAs. For each block the wave computes
// the transposed score tile
//     S^T[key, query] = K_tile . Q^T      (v_mfma_f32_32x32x16_bf16)
// so that in the MFMA accumulator layout each lane holds ONE query (column
// lane%32) and 16 keys per 32-key block: the row max and row sum are in-lane
// plus one exchange between the two lane halves. The probabilities stay in
// that layout and feed the second product directly as the B operand:
//     O^T[d, query] += V^T . P^T          (v_mfma_f32_32x32x16_bf16)
// whose accumulator again has one query per lane, so the online-softmax
// rescale is lane-local. V^T operands come from row-major V in LDS through
// the gfx950 transposing LDS read (ds_read_b64_tr_b16).
//
// MFMA 32x32x16 bf16 lane layout (checked on the device):
//   A (32 x 16): lane l holds row l%32, k-slots (l/32)*8 .. +7
//   B (16 x 32): lane l holds col l%32, k-slots (l/32)*8 .. +7
//   C (32 x 32): lane l holds col l%32, rows (i/4)*8 + (l/32)*4 + i%4, i < 16
// The k-slot -> key assignment of the PV product is free as long as A and B
// agree; it is chosen to match the C layout of S^T, so P needs no shuffle:
//   slot j of half h in PV step t  <->  key 16t + (j/4)*8 + 4h + j%4.
//
// Pipeline. K/V tiles move HBM -> LDS with direct-to-LDS loads (no register
// staging) into two buffers each. Iteration t computes S(t) = K(t) Q^T for
// both blocks, then issues O += P(t-1) V(t-1) on the MFMA pipe while the
// softmax of S(t) runs on the VALU; meanwhile K(t+1) and V(t) stream into the
// other buffers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_params.h"

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))
#define GLOBAL_AS __attribute__((address_space(1)))

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kQB = 1;                        // 32-query blocks per wave
constexpr int kRowsPerWave = 32 * kQB;        // query rows per wave
constexpr int kWavesPerSimd = kQB == 1 ? 2 : 1;  // occupancy the register budget allows

template <int D>
struct Tile {
  static constexpr int BN = (D == 128 && kQB > 1) ? 32 : 64;  // keys per tile
  static constexpr int NC = D / 8;                   // 16-byte chunks per K/V row
  static constexpr int KB = BN / 32;                 // 32-key blocks per tile
  static constexpr int DB = D / 32;                  // 32-wide d blocks of O^T
  static constexpr int QS = D / 16;                  // k-steps of the QK^T product
  static constexpr int PS = BN / 16;                 // k-steps of the PV product
  // LDS row pitches in 16-byte chunks (LDS: 64 banks x 4 bytes). K is read
  // 16 bytes per lane with consecutive lanes on consecutive rows: one pad
  // chunk staggers the rows by 4 banks, so 16 lanes cover all 64 banks. V is
  // read by the transposing load, where a half-wave touches 4 consecutive
  // rows x 64 bytes: four pad chunks put those rows 64 bytes apart modulo
  // 256. Either way every operand address is a per-lane base plus an
  // immediate.
  static constexpr int KPITCH = NC + 1;
  static constexpr int VPITCH = NC + 4;
  // Buffers are whole wave loads (64 chunks); chunks past the last row land
  // in the allocation's tail and are never read.
  static constexpr int KCHUNKS = (BN * KPITCH + 63) / 64 * 64;
  static constexpr int VCHUNKS = (BN * VPITCH + 63) / 64 * 64;
  static constexpr int KLOADS = KCHUNKS / 64;        // wave-wide loads per K tile
  static constexpr int VLOADS = VCHUNKS / 64;
  static constexpr int KPER = (KLOADS + kWaves - 1) / kWaves;  // per wave (upper bound)
  static constexpr int VPER = (VLOADS + kWaves - 1) / kWaves;
  static_assert(KPER <= 8 && VPER <= 8, "load offset tables hold 8 entries");
};

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

// Cross-half exchange: lanes l and l^32 hold the same query, different keys.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lazy rescaling: the running max used for the exponent is only moved when
// some row's max grew by more than 2^kTau (base 2); until then probabilities
// may exceed 1 by at most that factor, which bf16 and fp32 carry exactly as
// well. The final division by the row sum uses the same reference, so the
// result is unchanged up to rounding.
constexpr float kTau = 8.0f;

// Word 3 of a raw buffer descriptor (gfx9 family): 32-bit data format, no
// swizzle; with stride 0 an access is in range iff offset < num_records, and
// out-of-range loads return zero.
constexpr int kBufferWord3 = 0x00020000;

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMFMA = 0x008, kSchedDSRead = 0x100;

// s_waitcnt vmcnt(0): wait for this wave's direct-to-LDS loads.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, kWavesPerSimd) void attn_fwd_bf16_kernel(const Params p) {
  using TL = Tile<D>;
  constexpr int BN = TL::BN, NC = TL::NC, KB = TL::KB, DB = TL::DB, QS = TL::QS, PS = TL::PS;
  constexpr int KPITCH = TL::KPITCH, VPITCH = TL::VPITCH;

  // Four distinct LDS objects, so the compiler can tell that the loads in
  // flight into one buffer never alias reads of another.
  __shared__ u32x4 kbuf0[TL::KCHUNKS];
  __shared__ u32x4 kbuf1[TL::KCHUNKS];
  __shared__ u32x4 vbuf0[TL::VCHUNKS];
  __shared__ u32x4 vbuf1[TL::VCHUNKS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;   // k-slot half of the MFMA operands
  const int col = lane & 31;    // the query this lane owns
  const int il = lane & 15;     // index inside a 16-lane group (transposing read)
  const int grp = lane >> 4;    // 16-lane group

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
    h = r;
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

  // Per-lane byte offsets, inside a K/V tile, of the chunks this lane loads:
  // wave load n writes LDS chunks 64n .. 64n+63 (lane i -> chunk 64n + i);
  // chunk q of the padded tile is row q / pitch, column q % pitch, and pad
  // columns re-read column 0 of their row. Wave w issues loads w, w+4, ...
  uint32_t koff[TL::KPER], voff[TL::VPER];
#pragma unroll
  for (int j = 0; j < TL::KPER; ++j) {
    const int q = (wave + j * kWaves) * 64 + lane;
    const int r = q / KPITCH, cc = q % KPITCH;
    koff[j] = (uint32_t)(r * (D * 2) + (cc < NC ? cc : 0) * 16);
  }
#pragma unroll
  for (int j = 0; j < TL::VPER; ++j) {
    const int q = (wave + j * kWaves) * 64 + lane;
    const int r = q / VPITCH, cc = q % VPITCH;
    voff[j] = (uint32_t)(r * (D * 2) + (cc < NC ? cc : 0) * 16);
  }

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

    // keys a wave needs (causal rows r allow keys <= r)
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
    if (ntiles == 0) {
      if (active) {
        const int row = me.row0 + col;  // no valid key: output rows are 0
        if (row < p.Lq) {
          __bf16* orow = og + (q_head + row) * D;
          for (int d = half * (D / 2); d < (half + 1) * (D / 2); ++d) orow[d] = (__bf16)0.f;
        }
      }
      continue;
    }
    const int my_total = active ? (keys_needed(me) + BN - 1) / BN : 0;
    // tiles whose every key is valid for every row of this wave (no mask needed)
    int full_keys = nvalid;
    if (CAUSAL) full_keys = min(full_keys, me.row0 + 1);
    const int my_full = active ? min(full_keys / BN, my_total) : 0;

    const size_t kv_head = ((size_t)kvb * p.Hkv + g) * (size_t)p.Lk;
    const char* __restrict__ kg = (const char*)p.k + kv_head * (D * 2);
    const char* __restrict__ vg = (const char*)p.v + kv_head * (D * 2);

    // Direct-to-LDS buffer loads of tile t. The buffer descriptor spans this
    // (batch, head)'s Lk rows, so chunks of rows past the end read as zero
    // (those keys are masked or never read); the tile offset is a scalar.
    const uint32_t kv_bytes = (uint32_t)p.Lk * (D * 2);
    const __amdgpu_buffer_rsrc_t krsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)kg, (short)0, (int)kv_bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t vrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)vg, (short)0, (int)kv_bytes, kBufferWord3);
    auto load_tile = [&](__amdgpu_buffer_rsrc_t rsrc, u32x4* dst, int t, const uint32_t* off,
                         auto per_c, auto nloads_c) {
      constexpr int PER = decltype(per_c)::value, NLOADS = decltype(nloads_c)::value;
      const uint32_t tile_off = (uint32_t)t * (BN * D * 2);
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int n = wave + j * kWaves;
        if (j < PER - 1 || n < NLOADS)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void LDS_AS*)(dst + n * 64), 16, off[j],
                                                   tile_off, 0, 0);
      }
    };
    auto load_k = [&](u32x4* dst, int t) {
      load_tile(krsrc, dst, t, koff, std::integral_constant<int, TL::KPER>{},
                std::integral_constant<int, TL::KLOADS>{});
    };
    auto load_v = [&](u32x4* dst, int t) {
      load_tile(vrsrc, dst, t, voff, std::integral_constant<int, TL::VPER>{},
                std::integral_constant<int, TL::VLOADS>{});
    };

    // Q^T operands: block qb, lane holds query row0+32qb+col, d = 16*s + 8*half + 0..7.
    bf16x8 qreg[kQB][QS];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const int row = me.row0 + 32 * qb + col;
      const bool ok = active && row < p.Lq;
      const __bf16* qrow = qg + (q_head + (ok ? row : 0)) * D;
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (ok) x = *(const u32x4*)(qrow + 16 * s + 8 * half);
        qreg[qb][s] = __builtin_bit_cast(bf16x8, x);
      }
    }

    f32x16 oacc[kQB][DB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[qb][b][i] = 0.f;
    float m_run[kQB], l_run[kQB];   // reference max (raw scores) and this lane's partial sum
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      m_run[qb] = -INFINITY;
      l_run[qb] = 0.f;
    }
    bf16x8 pprev[kQB][PS];          // probabilities of the previous tile (PV operand)

    // S^T(t) = K(t) . Q^T for both blocks; each K operand feeds two MFMAs and
    // the next step's operands are read ahead.
    auto qk = [&](f32x16 (&sacc)[kQB][KB], const u32x4* kb) {
      const u32x4* kl = kb + col * KPITCH + half;
      bf16x8 a[2][KB];
#pragma unroll
      for (int kbk = 0; kbk < KB; ++kbk) {
        a[0][kbk] = __builtin_bit_cast(bf16x8, kl[kbk * 32 * KPITCH]);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[qb][kbk][i] = 0.f;
      }
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        if (s + 1 < QS) {
#pragma unroll
          for (int kbk = 0; kbk < KB; ++kbk)
            a[(s + 1) & 1][kbk] = __builtin_bit_cast(bf16x8, kl[kbk * 32 * KPITCH + 2 * (s + 1)]);
        }
#pragma unroll
        for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
            sacc[qb][kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 1][kbk], qreg[qb][s],
                                                                    sacc[qb][kbk], 0, 0, 0);
      }
      // Keep PF K operand reads in flight ahead of the MFMAs.
      constexpr int R = QS * KB, PF = R < 4 ? R : 4;
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, PF, 0);
#pragma unroll
      for (int i = 0; i < R - PF; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, kQB, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, kQB * PF, 0);
    };
    // O^T += V^T . P^T; V^T operands through the transposing LDS read:
    // source role il addresses V[row][dcol .. dcol+3], result lane il then
    // holds V[key0 + s][dbase + il] for s = 0..3. Next step read ahead.
    const int vlane = (half * 4 + (il >> 2)) * (VPITCH * 16) + ((grp & 1) * 16 + 4 * (il & 3)) * 2;
    auto pv = [&](const u32x4* vb32) {
      const LDS_AS char* vb = (const LDS_AS char*)vb32 + vlane;
      auto vread = [&](int ps, int b) -> bf16x8 {
        const int o1 = (ps * 16) * (VPITCH * 16) + b * 64;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(vb + o1));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4*)(vb + o1 + 8 * (VPITCH * 16)));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      bf16x8 a[2];
      a[0] = vread(0, 0);
#pragma unroll
      for (int step = 0; step < PS * DB; ++step) {
        const int ps = step / DB, b = step % DB;
        if (step + 1 < PS * DB) a[(step + 1) & 1] = vread((step + 1) / DB, (step + 1) % DB);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          oacc[qb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[step & 1], pprev[qb][ps],
                                                                oacc[qb][b], 0, 0, 0);
      }
      // Keep two steps (four transposing reads) in flight ahead of the MFMAs.
      constexpr int STEPS = PS * DB;
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 4, 0);
#pragma unroll
      for (int i = 0; i < STEPS - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, kQB, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 2 * kQB, 0);
    };
    // Online softmax of block qb for tile t (base 2, scale folded into c);
    // produces the next PV operand and returns the rescale factor of O.
    auto softmax = [&](f32x16 (&sacc)[KB], int qb, int t, bool masked, bf16x8 (&pout)[PS]) -> float {
      if (masked) {
        const int key0 = t * BN;
        const int qrow = me.row0 + 32 * qb + col;
#pragma unroll
        for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + kbk * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
            bool dead = key >= nvalid;
            if (CAUSAL) dead = dead || key > qrow;
            if (dead) sacc[kbk][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kbk][i]);
      mx = halves_max(mx);
      const float m_old = m_run[qb];
      const float m_new = fmaxf(m_old, mx);
      const bool grow = (m_new - m_old) * c > kTau;  // false for -inf - -inf (NaN)
      const bool move = __ballot(grow) != 0;
      const float m_use = move ? m_new : m_old;
      const float alpha = (!move || m_use == -INFINITY) ? 1.f
                                                        : __builtin_amdgcn_exp2f((m_old - m_use) * c);
      const float mc = (m_use == -INFINITY) ? 0.f : m_use * c;
      m_run[qb] = m_use;
      float rs = 0.f;
#pragma unroll
      for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kbk][i], c, -mc));
          sacc[kbk][i] = e;
          rs += e;
        }
      l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
      for (int ps = 0; ps < PS; ++ps)
#pragma unroll
        for (int j = 0; j < 8; ++j) pout[ps][j] = (__bf16)sacc[ps >> 1][(ps & 1) * 8 + j];
      return alpha;
    };
    auto rescale = [&](int qb, float alpha) {
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[qb][b][i] *= alpha;
      }
    };

    // ---- software-pipelined tile loop ----------------------------------------
    // Iteration t reads K(t) and V(t-1) while K(t+1) and V(t) stream into the
    // other buffers; the loop is unrolled by two so every access names one
    // fixed LDS buffer.
    f32x16 sacc[kQB][KB];
    auto iteration = [&](auto parity, int t) {
      constexpr int PAR = decltype(parity)::value;
      u32x4* kcur = PAR ? kbuf1 : kbuf0;
      u32x4* knext = PAR ? kbuf0 : kbuf1;
      u32x4* vprev = PAR ? vbuf0 : vbuf1;
      u32x4* vcur = PAR ? vbuf1 : vbuf0;
      if (t + 1 < ntiles) load_k(knext, t + 1);
      if (t < ntiles) load_v(vcur, t);
      if (active) {
        const bool do_pv = t >= 1 && t <= my_total;
        const bool do_sm = t < my_total;
        // Raise this wave's issue priority while it feeds the MFMA pipe, so
        // the other wave on the SIMD fills the gaps with its softmax VALU.
        if (do_sm) {
          __builtin_amdgcn_s_setprio(1);
          qk(sacc, kcur);
          __builtin_amdgcn_s_setprio(0);
        }
        if (do_pv) {
          __builtin_amdgcn_s_setprio(1);
          pv(vprev);
          __builtin_amdgcn_s_setprio(0);
        }
        if (do_sm) {
          const bool masked = t >= my_full;
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb) {
            bf16x8 pnew[PS];
            const float alpha = softmax(sacc[qb], qb, t, masked, pnew);
            rescale(qb, alpha);
#pragma unroll
            for (int ps = 0; ps < PS; ++ps) pprev[qb][ps] = pnew[ps];
          }
        }
      }
      wait_vm();
      __syncthreads();
    };
    load_k(kbuf0, 0);
    wait_vm();
    __syncthreads();
    int t = 0;
    for (; t + 1 <= ntiles; t += 2) {
      iteration(std::integral_constant<int, 0>{}, t);
      iteration(std::integral_constant<int, 1>{}, t + 1);
    }
    if (t <= ntiles) iteration(std::integral_constant<int, 0>{}, t);

    // ---- epilogue: O = O^T / l, round to bf16, store ---------------------------
    if (active) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const float l = halves_sum(l_run[qb]);
        const float inv = (l > 0.f) ? 1.f / l : 0.f;
        const int row = me.row0 + 32 * qb + col;
        if (row < p.Lq) {
          __bf16* orow = og + (q_head + row) * D;
#pragma unroll
          for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) {
              bf16x4 w;
#pragma unroll
              for (int j = 0; j < 4; ++j) w[j] = (__bf16)(oacc[qb][b][m4 * 4 + j] * inv);
              *(bf16x4*)(orow + b * 32 + m4 * 8 + half * 4) = w;
            }
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

// Work decomposition for the bf16 kernel: query rows are split into wave
// blocks of kRowsPerWave; a workgroup takes 4 consecutive blocks of one
// (batch entry, head), or, for short sequences, whole batch entries of
// 1, 2 or 4 blocks each (packed so a workgroup never straddles an entry).
bool plan_bf16(Params& p) {
  const int64_t nrb = ((int64_t)p.Lq + kRowsPerWave - 1) / kRowsPerWave;
  if (nrb >= kWaves) {
    p.P = (int)(((nrb + kWaves - 1) / kWaves) * kWaves);
    p.G = 1;
    p.nMT = p.P / kWaves;
    p.NG = p.NB;
  } else {
    p.P = (nrb == 3) ? 4 : (int)nrb;
    p.G = kWaves / p.P;
    p.nMT = 1;
    p.NG = (p.NB + p.G - 1) / p.G;
  }
  const int64_t T = (int64_t)p.NG * p.H * p.nMT;
  if (T > 0x7fffffff) return false;
  p.T = (int)T;
  // Keep all tiles that read one K/V head on one XCD (its L2), so each K/V
  // head streams from memory into a single L2. Broadcast tiles of one head
  // are ordered by candidate group; runs of 16 groups usually share a user.
  p.chunk = (p.cand2user == nullptr) ? p.nMT * (p.H / p.Hkv) : 16;
  return true;
}

}  // namespace attn
