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
// Work decomposition. A workgroup is 8 waves (two per SIMD); each wave owns
// 32 query rows of one (batch entry, head). The wave computes the transposed
// score tile
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
// The 8-wave d = 128 schedule uses MFMA 16x16x32 bf16 instead (it sustains a
// higher rate at the chip's power limit). Lane layout (checked on the device):
//   A (16 x 32): lane l holds row l%16, k-slots (l/16)*8 .. +7
//   B (32 x 16): lane l holds col l%16, k-slots (l/16)*8 .. +7
//   C (16 x 16): lane l holds col l%16, rows (l/16)*4 + i, i < 4
// A wave's 32 queries are two blocks of 16 (lane l holds query l%16 of each)
// and a key tile is four blocks of 16 (lane l holds keys 4(l/16) .. +3 of
// each); row reductions exchange across the four 16-lane rows. In PV step c
// (32 keys), slot j of row g  <->  key 32c + 4g + j (j < 4), 32c + 16 + 4g +
// j - 4 (j >= 4): key blocks 2c and 2c + 1 as the C layout holds them.
//
// Pipeline. K/V tiles move HBM -> LDS with direct-to-LDS buffer loads (no
// register staging) into two buffers each, shared by all 8 waves. The waves
// form two groups (waves 0-3 and 4-7; waves w and w+4 share a SIMD) that
// ping-pong in half-steps, with a workgroup barrier after every second one:
// while one group issues its MFMA phase for tile t (S(t) = K(t) Q^T and
// O += P(t-1) V(t-1)), the other runs the softmax of its previous tile on the
// VALU, so each SIMD's matrix pipe and vector ALU are busy at the same time.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "attn_params.h"

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kGroupWaves = 4;                // waves per ping-pong group (one per SIMD)
constexpr int kQB = 1;                        // 32-query blocks per wave
constexpr int kRowsPerWave = 32 * kQB;        // query rows per wave

template <int D, int W>
struct Tile {
  static constexpr int BN = (D == 128 && kQB > 1) ? 32 : 64;  // keys per tile
  static constexpr int NC = D / 8;                   // 16-byte chunks per K/V row
  static constexpr int KB = BN / 32;                 // 32-key blocks per tile
  static constexpr int DB = D / 32;                  // 32-wide d blocks of O^T
  static constexpr int QS = D / 16;                  // k-steps of the QK^T product
  static constexpr int PS = BN / 16;                 // k-steps of the PV product
  // LDS layouts (LDS: 64 banks x 4 bytes; a chunk is 16 bytes). Each wave
  // load fills one 1 KB window with 64 / NC whole rows of K or V, so that it
  // reads whole rows of memory, and neither layout has pad chunks to load.
  // K: window w holds rows w, w + NWIN, w + 2 NWIN, ... row-major, and the
  // windows start KWIN chunks apart: (row r, chunk c) is at chunk
  // (r % NWIN) * KWIN + (r / NWIN) * NC + c. A K operand read has 16 lanes on
  // 16 consecutive rows at one chunk; the one-chunk stagger of the windows
  // (and, at d = 64, the row offset inside a window) puts them on 16
  // distinct 16-byte bank groups. V: window n holds rows n * VROWS ..
  // n * VROWS + VROWS - 1, split into d-blocks of 32 columns, block-major:
  // window offset = block * VROWS * 64 + (row % VROWS) * 64 + byte. The
  // transposing read of a half-wave touches 4 consecutive rows x 64 bytes of
  // one block: 256 contiguous bytes, every bank once. Either way every
  // operand address is a per-lane base plus an immediate.
  static constexpr int NWIN = BN * NC / 64;          // K windows (= wave loads) per tile
  // chunks between K window starts: 65 for the 32 x 32 operand reads, 66 for
  // the 16 x 16 ones of the 8-wave d = 128 schedule. A 16-byte operand read
  // is served 32 lanes at a time over 512 bytes of banks (measured: a
  // pattern whose lane groups 0 and 1 sat 16 bytes apart had four conflict
  // cycles per read). There, lanes l and l + 16 read one row 16 bytes apart,
  // so consecutive rows must sit 32 bytes apart modulo 512: 66 chunks.
  static constexpr int KWIN = (W == 8 && D == 128) ? 66 : 65;
  static_assert(32 % NWIN == 0, "a 32-key block spans whole rounds of K windows");
  static constexpr int VROWS = 64 / NC;              // V rows per 1 KB window
  static_assert(VROWS == 4 || VROWS == 8, "a V read's 16-row step spans whole windows");
  static constexpr int KCHUNKS = NWIN * KWIN;
  static constexpr int VCHUNKS = BN * NC;
  static_assert(VCHUNKS % 64 == 0, "V tile is whole wave loads");
  // Unused chunks after each V buffer at d = 128. Measured: with a workgroup
  // LDS size of exactly 66 KB the two-per-CU 4-wave kernels ran the L = 2048
  // causal workload 4-5% slower than with any of 66 KB + 32 B, 68, 70, 72,
  // 74, 78 or 80 KB (same host, interleaved runs); the cause is not known.
  static constexpr int VSLACK = D == 128 ? 64 : 0;
  static constexpr int KLOADS = NWIN;                // wave-wide loads per K tile
  static constexpr int VLOADS = VCHUNKS / 64;
  static constexpr int KPER = (KLOADS + W - 1) / W;  // loads per wave (upper bound)
  static constexpr int VPER = (VLOADS + W - 1) / W;
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

// A wave-uniform 64-bit value, moved to scalar registers.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
  return ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)x);
}

struct WaveTask {
  int batch;   // query-side batch entry
  int row0;    // first query row of the wave
  int lq;      // query rows of the wave's sequence
  int kvb;     // K/V batch entry (user for the broadcast variant)
  bool valid;  // rows exist
  bool bad;    // kvb out of range: output NaN
};

// Maximum that propagates NaN. fmaxf must quiet signalling NaNs, so on
// values the compiler cannot prove canonical (MFMA results) every operand
// costs an extra self-max; this form maps to v_maximum3_f32 directly. A NaN
// score gives a NaN row either way, through the exponential.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Cross-half exchange: lanes l and l^32 hold the same query, different keys.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The same over the four 16-lane rows (lanes l, l^16, l^32, l^48 hold one
// query in the 16 x 16 tiles of v_mfma_f32_16x16x32_bf16): after the
// half exchange, one row-pair swap (rows 0 <-> 1, 2 <-> 3).
__device__ __forceinline__ float rowpair_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rowpair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float quarters_max(float x) { return rowpair_max(halves_max(x)); }
__device__ __forceinline__ float quarters_sum(float x) { return rowpair_sum(halves_sum(x)); }

// Lazy rescaling: the reference r used for the exponent 2^(u - r) moves to
// the row max on a row's first unmasked tile and then stays put while every
// probability it gives is at most 2^kTau (base 2), checked through the tile's
// partial row sums; probabilities may then exceed 1 by at most that factor,
// which bf16 and fp32 carry as well. The final division by the row sum uses
// the same reference, so the result is unchanged up to rounding. A reference
// at the row max makes the largest probability exactly 1, with no bf16
// rounding error against the fp32 row sum: rows dominated by one key keep
// that key's value exactly.
constexpr float kTau = 8.0f;
constexpr float kSumLimit = 256.0f;   // 2^kTau

// Word 3 of a raw buffer descriptor (gfx9 family): 32-bit data format, no
// swizzle; with stride 0 an access is in range iff offset < num_records, and
// out-of-range loads return zero.
constexpr int kBufferWord3 = 0x00020000;

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMFMA = 0x008, kSchedDSRead = 0x100;

// s_waitcnt vmcnt(0): wait for this wave's direct-to-LDS loads.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): wait until at most N of this wave's loads are in
// flight (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// W = 4: 4-wave workgroups (one wave per SIMD), the software-pipelined loop,
// two per CU at d = 128 and three at d = 64, whose 33 KB of LDS allow it and
// whose registers fit the three-per-CU budget (168 VGPRs) without spills: a
// third wave per SIMD hides more of the softmax, which at d = 64 weighs as
// much as the MFMA work. W = 8: one 8-wave workgroup per CU, the ping-pong
// loop (waves w and w+4 on one SIMD).
template <int D, int W>
constexpr int kGroupsPerCU = W == 4 ? (D == 64 ? 3 : 2) : 1;
// Tensor layouts of the kernel instantiations.
constexpr int kDense = 0, kJagged = 1, kSparse = 2;
// Most key blocks a block-sparse query block may list (LDS list size).
constexpr int kMaxKeyBlocks = 1024;

template <int D, bool CAUSAL, int W, int LAYOUT>
__global__ __launch_bounds__(W * 64, (kGroupsPerCU<D, W>)) void attn_fwd_bf16_kernel(const Params p) {
  using TL = Tile<D, W>;
  constexpr int kWaves = W;
  constexpr int BN = TL::BN, NC = TL::NC;
  // Matrix-core shape. The 8-wave d = 128 schedule runs both products on
  // v_mfma_f32_16x16x32_bf16: on this chip, at the power limit, it sustains
  // about 1.5 times the rate of v_mfma_f32_32x32x16_bf16 on the same operand
  // data (half the accumulator traffic per FLOP). Its 16 x 16 tiles put a
  // wave's 32 queries in two blocks of 16 (lane l holds query l % 16 of each)
  // and a tile's keys in blocks of 16 (lane l holds keys 4 (l / 16) .. +3 of
  // each); the other schedules keep the 32 x 32 tiles: one block of 32
  // queries (lane l holds query l % 32) and keys in blocks of 32.
  constexpr bool M16 = W == 8 && D == 128;
  constexpr int QB = M16 ? 2 : kQB;               // query blocks per wave
  constexpr int QR = M16 ? 16 : 32;               // queries per block
  constexpr int KB = M16 ? BN / 16 : TL::KB;      // key blocks per tile
  constexpr int DB = M16 ? D / 16 : TL::DB;       // d blocks of O^T
  constexpr int QS = M16 ? D / 32 : TL::QS;       // k-steps of the QK^T product
  constexpr int PS = M16 ? BN / 32 : TL::PS;      // k-steps of the PV product
  constexpr int AE = M16 ? 4 : 16;                // accumulator floats per lane
  using Acc = std::conditional_t<M16, f32x4, f32x16>;
  // Chunks between V window starts. The 16 x 16 transposing reads of lane
  // groups 0 and 1 (and 2 and 3) fall on consecutive windows, so the windows
  // are staggered by 32 bytes there (within the slack of the V buffers), which
  // puts the two groups of a read cycle on different banks.
  constexpr int VWIN = M16 ? 66 : 64;
  static_assert(TL::VLOADS * VWIN <= TL::VCHUNKS + TL::VSLACK, "staggered V windows fit the buffer");
  constexpr int NWIN = TL::NWIN, KWIN = TL::KWIN, VROWS = TL::VROWS;

  // Four distinct LDS objects, so the compiler can tell that the loads in
  // flight into one buffer never alias reads of another.
  __shared__ u32x4 kbuf0[TL::KCHUNKS];
  __shared__ u32x4 kbuf1[TL::KCHUNKS];
  __shared__ u32x4 vbuf0[TL::VCHUNKS + TL::VSLACK];
  __shared__ u32x4 vbuf1[TL::VCHUNKS + TL::VSLACK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;   // k-slot half of the MFMA operands
  const int col = lane & 31;    // the query this lane owns
  const int il = lane & 15;     // index inside a 16-lane group (transposing read)
  const int grp = lane >> 4;    // 16-lane group
  const int qcol = M16 ? il : col;   // the query of a block this lane holds
  const int qgrp = M16 ? grp : half; // which keys of a key block it holds

  // ---- decode the logical tile --------------------------------------------
  const int L = xcd_remap(blockIdx.x, p.T, p.chunk);
  const int HPG = p.H / p.Hkv;
  int bgrp, h, mt;
  if (p.cand2user == nullptr) {
    // dense: chunks of p.units (batch group, K/V head) units, ordered inside as
    // (mt' * units + unit) * HPG + hq, so a causal chunk runs the heaviest row
    // block of every unit first (longest-first over the XCD's share); the
    // last chunk may hold fewer units.
    const int per_chunk = p.units * p.nMT * HPG;
    const int sup = L / per_chunk;
    const int nu = min(p.units, p.NG * p.Hkv - sup * p.units);
    const int r0 = L - sup * per_chunk;
    const int hq = r0 % HPG;
    const int r = r0 / HPG;
    const int unit = sup * p.units + r % nu;
    const int mtr = r / nu;
    const int g = unit % p.Hkv;
    bgrp = unit / p.Hkv;
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

  // Row addressing. Dense: rows of one (batch, head) are contiguous, D
  // elements apart. Jagged (a separate instantiation, so the dense kernels
  // keep compile-time strides): tokens are packed [total, heads, D], so rows
  // of one head are heads*D elements apart and sequence b starts at token
  // offsets[b]; lengths come from the offsets, clamped to [0, Lq] / [0, Lk].
  constexpr bool jagged = LAYOUT == kJagged;
  constexpr bool sparse = LAYOUT == kSparse;
  // block-sparse: active key blocks of the workgroup's query block, then the count
  __shared__ int klist[sparse ? kMaxKeyBlocks + 1 : 1];
  const int q_rs = jagged ? p.H * D : D;
  const int kv_rs = jagged ? p.Hkv * D : D;
  auto seq_len = [&](const int32_t* off, int b, int cap) __attribute__((always_inline)) -> int {
    return min(max(off[b + 1] - off[b], 0), cap);
  };

  // The tasks of all waves, computed together (every thread derives every
  // wave's task: the pass loop bounds are shared). Each level of indirection
  // (the slot order, the jagged offsets, cand2user) loads the entries of all
  // waves before any is used, so the chain costs one round trip per level
  // rather than one per wave and level. Indices are clamped, so the loads stay
  // in bounds whatever the batch index.
  WaveTask tk[kWaves];
  int bcl[kWaves];
  bool in_range[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (p.G == 1) {
      tk[w].batch = bgrp;
      tk[w].row0 = (mt * kWaves + w) * kRowsPerWave;
    } else {
      tk[w].batch = bgrp * p.G + w / p.P;
      tk[w].row0 = (w % p.P) * kRowsPerWave;
    }
    bcl[w] = min(tk[w].batch, p.NB - 1);
    in_range[w] = tk[w].batch < p.NB;
  }
  if (p.cand_order != nullptr) {
    // broadcast with a slot order: the slot's candidate (out of range: no rows)
    int cand[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) cand[w] = p.cand_order[bcl[w]];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      tk[w].batch = cand[w];
      in_range[w] = in_range[w] && (unsigned)cand[w] < (unsigned)p.NB;
    }
  }
  if constexpr (jagged) {
    int lo[kWaves], hi[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      lo[w] = p.q_offsets[bcl[w]];
      hi[w] = p.q_offsets[bcl[w] + 1];
    }
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tk[w].lq = min(max(hi[w] - lo[w], 0), p.Lq);
  } else {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tk[w].lq = p.Lq;
  }
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    tk[w].valid = in_range[w] && tk[w].row0 < tk[w].lq;
    tk[w].kvb = tk[w].batch;
    tk[w].bad = false;
  }
  // The wave's own rows are wave-uniform; moving them to scalar registers lets
  // the compiler treat everything derived from them (loop bounds, buffer
  // descriptors) as uniform.
  WaveTask me = tk[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w)
    if (wave == w) me = tk[w];
  me.batch = __builtin_amdgcn_readfirstlane(me.batch);
  me.row0 = __builtin_amdgcn_readfirstlane(me.row0);
  me.lq = __builtin_amdgcn_readfirstlane(me.lq);
  me.valid = __builtin_amdgcn_readfirstlane((int)me.valid) != 0;
  // element offset of row 0 of this wave's (sequence, head)
  size_t q_base = ((size_t)(me.valid ? me.batch : 0) * p.H + h) * (size_t)p.Lq * D;
  if (jagged) q_base = me.valid ? (size_t)p.q_offsets[me.batch] * q_rs + (size_t)h * D : 0;
  const __bf16* __restrict__ qg = (const __bf16*)p.q + q_base;
  __bf16* __restrict__ og = (__bf16*)p.o + q_base;

  // The query rows next: they need no K/V index, so their round trip overlaps
  // the user lookup and the pass setup. A wave computes in exactly one pass.
  // Q^T operands: block qb, lane holds query row0+32qb+col, d = 16*s + 8*half + 0..7.
  // (16 x 16 tiles: lane l holds query row0+16qb+l%16, d = 32*s + 8*(l/16) + 0..7.)
  bf16x8 qreg[QB][QS];
  constexpr int QSTEP = M16 ? 32 : 16;   // d per k-step
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = me.row0 + QR * qb + qcol;
    const bool ok = me.valid && row < me.lq;
    const __bf16* qrow = qg + (size_t)(ok ? row : 0) * q_rs;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (ok) x = *(const u32x4*)(qrow + QSTEP * s + 8 * qgrp);
      qreg[qb][s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  if (p.cand2user != nullptr) {
    int u[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      u[w] = p.cand2user[p.cand_order != nullptr ? (in_range[w] ? tk[w].batch : 0) : bcl[w]];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      tk[w].kvb = u[w];
      tk[w].bad = tk[w].valid && ((u[w] < 0) || (u[w] >= p.NKV));
    }
  }

  // the wave's K/V batch and user check, once the map is read
  {
    int kvb_me = tk[0].kvb;
    bool bad_me = tk[0].bad;
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
      if (wave == w) { kvb_me = tk[w].kvb; bad_me = tk[w].bad; }
    me.kvb = __builtin_amdgcn_readfirstlane(kvb_me);
    me.bad = __builtin_amdgcn_readfirstlane((int)bad_me) != 0;
  }

  // Candidates with an out-of-range user index get NaN rows.
  if (me.valid && me.bad) {
    const int row = me.row0 + col;
    if (row < me.lq) {
      __bf16* orow = og + (size_t)row * q_rs;
      const __bf16 nanv = __builtin_bit_cast(__bf16, (unsigned short)0x7FC0);
      for (int d = half * (D / 2); d < (half + 1) * (D / 2); ++d) orow[d] = nanv;
    }
  }

  const float c = p.c;

  // The pass leads: the first wave of each distinct K/V batch among the valid
  // ones (one pass per lead; normally exactly one).
  uint32_t leads = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    bool first = tk[w].valid && !tk[w].bad;
#pragma unroll
    for (int v = 0; v < w; ++v)
      first = first && !(tk[v].valid && !tk[v].bad && tk[v].kvb == tk[w].kvb);
    leads |= (uint32_t)first << w;
  }
  leads = __builtin_amdgcn_readfirstlane(leads);

  // Per-lane byte offsets, inside a K/V tile, of the chunks this lane loads
  // (wave load n fills window n, lane i its 16-byte slot i). K: lane i takes
  // row n + NWIN * (i / NC), column chunk i % NC. V: lane i takes d-block
  // i / (4 VROWS), row n * VROWS + (i / 4) % VROWS, column chunk
  // 4 * block + i % 4. Wave w issues loads w, w+W, ... (Unsigned arithmetic:
  // it compiles to shifts and adds.)
  uint32_t koff[TL::KPER], voff[TL::VPER];
  const uint32_t row_bytes = (uint32_t)kv_rs * 2u;
  const uint32_t ulane = (uint32_t)lane;
  const uint32_t kpart = (ulane / (uint32_t)NC) * (uint32_t)NWIN * row_bytes + (ulane % (uint32_t)NC) * 16u;
#pragma unroll
  for (int j = 0; j < TL::KPER; ++j) koff[j] = (uint32_t)(wave + j * kWaves) * row_bytes + kpart;
  const uint32_t vpart = ((ulane / 4u) % (uint32_t)VROWS) * row_bytes +
                         ((ulane / (4u * VROWS)) * 4u + ulane % 4u) * 16u;
#pragma unroll
  for (int j = 0; j < TL::VPER; ++j)
    voff[j] = (uint32_t)(wave + j * kWaves) * ((uint32_t)VROWS * row_bytes) + vpart;

  // One pass per distinct K/V batch among the waves.
  // A pass after the first reloads its query rows, and the registers are
  // declared undefined at the end of each pass (an empty asm that writes
  // them), so the rows are not kept live through a pass's epilogue for a
  // later pass.
  auto forget_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int s = 0; s < QS; ++s) asm volatile("" : "=v"(qreg[qb][s]));
  };
  bool first_pass = true;
  for (; leads != 0; forget_q(), first_pass = false, leads &= leads - 1) {
    const int lead = __builtin_ctz(leads);
    int kvb = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (w == lead) kvb = tk[w].kvb;
    kvb = __builtin_amdgcn_readfirstlane(kvb);
    const bool active = __builtin_amdgcn_readfirstlane(me.valid && !me.bad && me.kvb == kvb) != 0;
    if (!first_pass) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int row = me.row0 + QR * qb + qcol;
        const bool ok = active && row < me.lq;
        const __bf16* qrow = qg + (size_t)(ok ? row : 0) * q_rs;
#pragma unroll
        for (int s = 0; s < QS; ++s) {
          u32x4 x = {0u, 0u, 0u, 0u};
          if (ok) x = *(const u32x4*)(qrow + QSTEP * s + 8 * qgrp);
          qreg[qb][s] = __builtin_bit_cast(bf16x8, x);
        }
      }
    }

    int nvalid = jagged ? seq_len(p.kv_offsets, kvb, p.Lk) : p.Lk;
    if (p.kv_len != nullptr) nvalid = min(max(p.kv_len[kvb], 0), p.Lk);

    // keys a wave needs (causal rows r allow keys <= r)
    auto keys_needed = [&](const WaveTask& t) __attribute__((always_inline)) -> int {
      int n = nvalid;
      if (CAUSAL) n = min(n, min(t.row0 + kRowsPerWave, t.lq));
      return n;
    };
    // The key tiles of the pass, in order. Dense and jagged: 0, 1, 2, ...
    // Block-sparse: the tiles of the key blocks set in the mask row of the
    // workgroup's query block (every wave of a workgroup lies in one query
    // block: blk is a multiple of the workgroup's rows), compacted by wave 0.
    int nact = 0;
    int tpb = 1;   // tiles per key block
    if constexpr (sparse) {
      tpb = p.blk / BN;
      const int qblk = min(tk[0].row0 / p.blk, p.nQB - 1);
      const int hm = p.mask_heads == 1 ? 0 : h;
      if (wave == 0) {
        const uint8_t* mrow = p.block_mask + ((size_t)hm * p.nQB + qblk) * p.nKB;
        int cnt = 0;
        for (int base = 0; base < p.nKB; base += 64) {
          const int kb = base + lane;
          const bool on = kb < p.nKB && mrow[kb] != 0;
          const uint64_t bal = __ballot(on);
          const int before = __builtin_amdgcn_mbcnt_hi(
              (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
          if (on) klist[cnt + before] = kb;
          cnt += __builtin_popcountll(bal);
        }
        if (lane == 0) klist[kMaxKeyBlocks] = cnt;
      }
      __syncthreads();
      nact = __builtin_amdgcn_readfirstlane(klist[kMaxKeyBlocks]);
    }
    auto tile_of = [&](int s) __attribute__((always_inline)) -> int {
      if constexpr (sparse)
        return __builtin_amdgcn_readfirstlane(klist[s / tpb]) * tpb + s % tpb;
      else
        return s;
    };
    // tiles of the sequence with some key below `keys`, and with every key below it
    auto tiles_touching = [&](int keys) __attribute__((always_inline)) -> int {
      if constexpr (!sparse) {
        return (keys + BN - 1) / BN;
      } else {
        int n = 0;
        for (int i = 0; i < nact; ++i)
          n += min(max((keys - klist[i] * p.blk + BN - 1) / BN, 0), tpb);
        return n;
      }
    };
    auto tiles_inside = [&](int keys) __attribute__((always_inline)) -> int {
      if constexpr (!sparse) {
        return keys / BN;
      } else {
        int n = 0;
        for (int i = 0; i < nact; ++i) n += min(max((keys - klist[i] * p.blk) / BN, 0), tpb);
        return n;
      }
    };

    int ntiles = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const WaveTask& t = tk[w];
      if (t.valid && !t.bad && t.kvb == kvb) ntiles = max(ntiles, tiles_touching(keys_needed(t)));
    }
    ntiles = __builtin_amdgcn_readfirstlane(ntiles);
    if (ntiles == 0) {
      if (active) {
        const int row = me.row0 + col;  // no valid key: output rows are 0
        if (row < me.lq) {
          __bf16* orow = og + (size_t)row * q_rs;
          for (int d = half * (D / 2); d < (half + 1) * (D / 2); ++d) orow[d] = (__bf16)0.f;
        }
      }
      continue;
    }
    // Per-wave tile counts are wave-uniform; readfirstlane says so to the
    // compiler, so that branches on them stay scalar branches.
    const int my_total =
        __builtin_amdgcn_readfirstlane(active ? tiles_touching(keys_needed(me)) : 0);
    // tiles whose every key is valid for every row of this wave (no mask
    // needed); with tiles in increasing key order they come first
    int full_keys = nvalid;
    if (CAUSAL) full_keys = min(full_keys, me.row0 + 1);
    const int my_full =
        __builtin_amdgcn_readfirstlane(active ? min(tiles_inside(full_keys), my_total) : 0);

    size_t kv_base = ((size_t)kvb * p.Hkv + g) * (size_t)p.Lk * D;   // elements
    if (jagged) kv_base = (size_t)p.kv_offsets[kvb] * kv_rs + (size_t)g * D;
    const char* __restrict__ kg = (const char*)p.k + kv_base * 2;
    const char* __restrict__ vg = (const char*)p.v + kv_base * 2;

    // Direct-to-LDS buffer loads of tile t. Each tile gets its own buffer
    // descriptor: the base is the tile's first row and the range is the bytes
    // of this (batch, head)'s valid rows (the first nvalid: Lk, kv_len or the
    // sequence's length) from there on (none for a tile past the end). A
    // lane's only offset is its own chunk offset, so the range check is the
    // plain per-lane one: chunks of rows past the last valid one read as zero.
    // Those keys are masked, and their zero V rows
    // keep P = 0 times V at zero whatever the memory there holds (padding past
    // kv_len may be uninitialised: 0 * NaN would poison the row). The range
    // ends with the last valid row's own D elements, so later rows (other
    // heads or sequences in the jagged layout) are never read either.
    // The pass's K/V base addresses and valid byte range are wave-uniform:
    // kept in scalar registers, the per-tile descriptor is scalar arithmetic
    // (a descriptor the compiler cannot prove uniform costs a loop per load).
    const uint32_t kv_bytes = __builtin_amdgcn_readfirstlane(
        nvalid > 0 ? (uint32_t)(nvalid - 1) * (kv_rs * 2) + D * 2 : 0u);
    const uint64_t kaddr = uniform_u64((uint64_t)(uintptr_t)kg);
    const uint64_t vaddr = uniform_u64((uint64_t)(uintptr_t)vg);
    auto load_tile = [&](uint64_t base, u32x4* dst, int t, const uint32_t* off, auto per_c,
                         auto nloads_c, auto stride_c) __attribute__((always_inline)) {
      constexpr int PER = decltype(per_c)::value, NLOADS = decltype(nloads_c)::value;
      constexpr int STRIDE = decltype(stride_c)::value;   // chunks between windows
      const uint32_t tile_off = (uint32_t)t * (uint32_t)(BN * kv_rs * 2);
      // both below 2^31: a signed max, which has a scalar instruction (an
      // unsigned saturating subtract would go to a vector register)
      const int left = max((int)kv_bytes - (int)tile_off, 0);
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(uintptr_t)(base + tile_off), (short)0, left, kBufferWord3);
      // LDS destination of load j: the buffer's address plus this wave's
      // window offset plus a compile-time step. The wave offset passes through
      // an empty asm on every call, so the sum is one scalar add here rather
      // than one loop-invariant register per (buffer, j) pair, which the
      // compiler spilled to VGPR lanes and read back in the loops.
      uint32_t wofs = (uint32_t)wave * (uint32_t)(STRIDE * 16);
      asm volatile("" : "+s"(wofs));
      const uint32_t d0 = (uint32_t)(uintptr_t)((void LDS_AS*)dst) + wofs;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int n = wave + j * kWaves;
        if (j < PER - 1 || NLOADS % kWaves == 0 || n < NLOADS)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rsrc, (void LDS_AS*)(uintptr_t)(d0 + (uint32_t)(j * kWaves * STRIDE * 16)), 16, off[j],
              0, 0, 0);
      }
    };
    auto load_k = [&](u32x4* dst, int t) __attribute__((always_inline)) {
      load_tile(kaddr, dst, t, koff, std::integral_constant<int, TL::KPER>{},
                std::integral_constant<int, TL::KLOADS>{}, std::integral_constant<int, KWIN>{});
    };
    auto load_v = [&](u32x4* dst, int t) __attribute__((always_inline)) {
      load_tile(vaddr, dst, t, voff, std::integral_constant<int, TL::VPER>{},
                std::integral_constant<int, TL::VLOADS>{}, std::integral_constant<int, VWIN>{});
    };
    // Scaling (or normalising) the queries waits for their loads; each
    // schedule calls this after issuing its first K/V tile loads, so that the
    // query and K/V round trips overlap.
    auto prep_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // The softmax scale c = scale * log2(e) is folded into the query
      // operands (one bf16 rounding of c * q), so the score MFMAs produce
      // base-2 logits directly. RMS normalisation of the query row is fused
      // the same way: the normalised queries never leave registers (the two
      // lane halves, or with 16 x 16 tiles the four 16-lane rows, hold the parts
      // of the row).
      if (!p.qnorm) {
#pragma unroll
        for (int s = 0; s < QS; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) qreg[qb][s][e] = (__bf16)((float)qreg[qb][s][e] * c);
      } else {
        float ss = 0.f;
#pragma unroll
        for (int s = 0; s < QS; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = (float)qreg[qb][s][e];
            ss = __builtin_fmaf(v, v, ss);
          }
        ss = M16 ? quarters_sum(ss) : halves_sum(ss);
        const float r = 1.0f / sqrtf(ss * (1.0f / D) + p.eps);
        // gamma_q (16-byte aligned) in 16-byte loads, all issued before any
        // is used; one branch for the whole row
        const float* __restrict__ gq = p.gamma_q;
        f32x4 g[QS][2];
        if (gq != nullptr) {
#pragma unroll
          for (int s = 0; s < QS; ++s)
#pragma unroll
            for (int k4 = 0; k4 < 2; ++k4) g[s][k4] = *(const f32x4*)(gq + QSTEP * s + 8 * qgrp + 4 * k4);
        } else {
#pragma unroll
          for (int s = 0; s < QS; ++s)
#pragma unroll
            for (int k4 = 0; k4 < 2; ++k4) g[s][k4] = f32x4{1.f, 1.f, 1.f, 1.f};
        }
#pragma unroll
        for (int s = 0; s < QS; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            qreg[qb][s][e] = (__bf16)((float)qreg[qb][s][e] * r * (g[s][e >> 2][e & 3] * c));
      }
    }
    };

    Acc oacc[QB][DB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int i = 0; i < AE; ++i) oacc[qb][b][i] = 0.f;
    // Online-softmax state of the lane's query row, in base-2 logit units u
    // (the queries carry the scale): the reference r (scores are
    // exponentiated as 2^(u - r)), this lane's partial row sum, and pen =
    // +inf while the row has seen no unmasked key (0 after), which sends the
    // first tile through the exact path. -r replicated over one accumulator
    // block is the starting value of the score MFMAs, which then produce
    // u - r directly, so the exponent needs no subtraction. The 4-wave
    // schedules keep that block (16 registers) across the loop; the 8-wave
    // one has no registers to spare and writes it from r before each score
    // product, into registers that hold nothing live at that point.
    constexpr bool kSeed = true;
    constexpr bool kKeepSeed = W == 4;
    float r_ref[QB], l_run[QB], pen[QB];
    Acc neg_r[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      r_ref[qb] = 0.f;
      l_run[qb] = 0.f;
      pen[qb] = INFINITY;
#pragma unroll
      for (int i = 0; i < AE; ++i) neg_r[qb][i] = 0.f;
    }
    bf16x8 pprev[QB][PS];          // probabilities of the previous tile (PV operand)

    // V^T operands come through the transposing LDS read: source role il
    // addresses V[row][dcol .. dcol+3], result lane il then holds
    // V[key0 + s][dbase + il] for s = 0..3.
    // 32 x 32 tiles: group grp reads keys half*4 (+8) at d-columns (grp&1)*16 of
    // a 32-wide block. 16 x 16 tiles: group grp reads keys 4 grp (+16) at
    // d-columns 0..15 of a 16-wide block (V window grp, VROWS = 4).
    const int vrow = M16 ? 4 * grp + (il >> 2) : half * 4 + (il >> 2);
    const int vlane = M16 ? (vrow / VROWS) * (VWIN * 16) + (vrow % VROWS) * 64 + (il & 3) * 8
                          : (vrow / VROWS) * 1024 + (vrow % VROWS) * 64 + ((grp & 1) * 16 + 4 * (il & 3)) * 2;
    // Both products of one step in a single instruction stream: first
    // O += P(t-1) V(t-1), then S(t) = K(t) Q^T, so P(t-1) is dead before S(t)
    // is born. Operand reads run two MFMAs ahead through the whole stream
    // (a V^T operand is two reads, a K operand one), so the matrix pipe does
    // not wait at the seam between the products. PV_C / QK_C (compile time)
    // drop one of the products: the first tile of a pass has no PV product
    // and the step after the last tile no QK product.
    auto pvqk = [&](Acc (&sacc)[QB][KB], const u32x4* kb, const u32x4* vb32, auto pv_c,
                    auto qk_c) __attribute__((always_inline)) {
      constexpr bool PV = decltype(pv_c)::value, QK = decltype(qk_c)::value;
      if constexpr (M16) {
        static_assert(VROWS == 4 && NWIN == 16 && NC == 16, "16 x 16 tiles: d = 128 layouts");
        // K operand (key block kt, k-step s): lane l reads key kt*16 + l%16
        // (window l%16), chunk 4 s + l/16.
        const u32x4* kl = kb + il * KWIN + grp;
        const LDS_AS char* vb = (const LDS_AS char*)vb32 + vlane;
        constexpr int NK = QS * KB, NV = PS * DB;
        bf16x8 ka[QS][KB], va[NV];
        if constexpr (PV) {
          // V^T operand (32-key step c, 16-wide d block db): keys 32c + 4 grp
          // + 0..3 (lo) and 32c + 16 + 4 grp + 0..3 (hi) at d = 16 db + l%16,
          // matching the probabilities' k order.
#pragma unroll
          for (int step = 0; step < NV; ++step) {
            const int c = step / DB, db = step % DB;
            const int o1 = (c * 8) * (VWIN * 16) + (db / 2) * (VROWS * 64) + (db % 2) * 32;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(vb + o1));
            const bf16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(vb + o1 + 4 * (VWIN * 16)));
            va[step] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
#pragma unroll
          for (int step = 0; step < NV; ++step)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              oacc[qb][step % DB] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  va[step], pprev[qb][step / DB], oacc[qb][step % DB], 0, 0, 0);
        }
        if constexpr (QK) {
          Acc seed[QB];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int i = 0; i < AE; ++i) seed[qb][i] = -r_ref[qb];
#pragma unroll
          for (int s = 0; s < QS; ++s)
#pragma unroll
            for (int kt = 0; kt < KB; ++kt) ka[s][kt] = __builtin_bit_cast(bf16x8, kl[kt * NC + 4 * s]);
#pragma unroll
          for (int s = 0; s < QS; ++s)
#pragma unroll
            for (int kt = 0; kt < KB; ++kt)
#pragma unroll
              for (int qb = 0; qb < QB; ++qb)
                sacc[qb][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    ka[s][kt], qreg[qb][s], s > 0 ? sacc[qb][kt] : seed[qb], 0, 0, 0);
        }
        // operand reads two MFMA pairs ahead, as below
        if constexpr (PV && QK) {
          __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 4, 0);
#pragma unroll
          for (int i = 0; i < NV - 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, QB, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
          }
#pragma unroll
          for (int i = 0; i < NK; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, QB, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 2 * QB, 0);
        } else if constexpr (PV) {
          __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 4, 0);
#pragma unroll
          for (int i = 0; i < NV - 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, QB, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 2 * QB, 0);
        } else if constexpr (QK) {
          __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
#pragma unroll
          for (int i = 0; i < NK - 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, QB, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 2 * QB, 0);
        }
      } else {
      static_assert(QB == 1, "one query block per wave");
      const u32x4* kl = kb + (col % NWIN) * KWIN + (col / NWIN) * NC + half;
      const LDS_AS char* vb = (const LDS_AS char*)vb32 + vlane;
      constexpr int NK = QS * KB, NV = PS * DB;
      bf16x8 ka[QS][KB], va[NV];
      if constexpr (PV) {
#pragma unroll
        for (int step = 0; step < NV; ++step) {
          const int o1 = ((step / DB) * 16 / VROWS) * 1024 + (step % DB) * (VROWS * 64);
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(vb + o1));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (LDS_AS bf16x4*)(vb + o1 + (8 / VROWS) * 1024));
          va[step] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int step = 0; step < NV; ++step)
          oacc[0][step % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              va[step], pprev[0][step / DB], oacc[0][step % DB], 0, 0, 0);
      }
      if constexpr (QK) {
        f32x16 seed;
        if constexpr (kKeepSeed) {
          seed = neg_r[0];
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) seed[i] = -r_ref[0];
        }
#pragma unroll
        for (int s = 0; s < QS; ++s)
#pragma unroll
          for (int kbk = 0; kbk < KB; ++kbk)
            ka[s][kbk] = __builtin_bit_cast(bf16x8, kl[kbk * (32 / NWIN) * NC + 2 * s]);
#pragma unroll
        for (int s = 0; s < QS; ++s)
#pragma unroll
          for (int kbk = 0; kbk < KB; ++kbk)
            sacc[0][kbk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                ka[s][kbk], qreg[0][s], s > 0 ? sacc[0][kbk] : seed, 0, 0, 0);
      }
      if constexpr (PV && QK) {
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 4, 0);
#pragma unroll
        for (int i = 0; i < NV - 2; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
        }
#pragma unroll
        for (int i = 0; i < NK; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 2, 0);
      } else if constexpr (PV) {
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 4, 0);
#pragma unroll
        for (int i = 0; i < NV - 2; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 2, 0);
      } else if constexpr (QK) {
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
#pragma unroll
        for (int i = 0; i < NK - 2; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 2, 0);
      }
      }
    };
    using kOn = std::true_type;
    using kOff = std::false_type;
    // Online softmax of block qb for tile t: sacc holds u - r, the base-2
    // logits relative to the row's reference; produces the next PV operand
    // and returns the rescale factor of O.
    auto softmax = [&](Acc (&sacc)[KB], int qb, int tile, bool masked, bf16x8 (&pout)[PS]) __attribute__((always_inline)) -> float {
      if (masked) {
        // Element (kbk, i) holds key tile*BN + half*4 + off with a compile-time
        // off; it is dead (past kv_len, or after the row's own position when
        // causal) iff off >= lim. lim depends on the tile, so no comparison is
        // hoisted out of the tile loop as a loop-invariant mask.
        const int qrow = me.row0 + QR * qb + qcol;
        const int lim = (CAUSAL ? min(nvalid, qrow + 1) : nvalid) - (tile * BN + qgrp * 4);
#pragma unroll
        for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
          for (int i = 0; i < AE; ++i) {
            // 32 x 32: key 32 kbk + 8 (i / 4) + 4 half + i % 4;
            // 16 x 16: key 16 kbk + 4 grp + i
            const int off = M16 ? kbk * 16 + i : kbk * 32 + (i >> 2) * 8 + (i & 3);
            if (off >= lim) sacc[kbk][i] = -INFINITY;
          }
      }
      // Exponentials 2^(sacc - d), rounded to bf16 as the next PV operand;
      // returns this lane's partial row sum (fp32), started at `first`.
      auto exps = [&](auto shifted_c, float d, float first) __attribute__((always_inline)) -> float {
        float ps4[4] = {first, 0.f, 0.f, 0.f};   // four independent partial sums
#pragma unroll
        for (int ps = 0; ps < PS; ++ps)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            // the PV operand's k order: 32 x 32, keys of step ps from block ps/2;
            // 16 x 16, slots 0-3 from key block 2 ps, 4-7 from 2 ps + 1
            float x = M16 ? sacc[2 * ps + (j >> 2)][j & 3] : sacc[ps >> 1][(ps & 1) * 8 + j];
            if constexpr (decltype(shifted_c)::value) x -= d;
            const float e = __builtin_amdgcn_exp2f(x);
            ps4[j & 3] += e;
            pout[ps][j] = (__bf16)e;
          }
        return (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
      };
      // sacc holds u - r (seeded) or u; shift: what the exponent subtracts
      const float shift = kSeed ? 0.f : r_ref[qb];
      // Fast path: keep the current reference. Every probability is at most
      // its lane's partial sum, so if no lane's sum exceeds 2^kTau the tile
      // is done without forming the row max and O needs no rescale. A row
      // that has seen no unmasked key starts its sum at +inf and falls
      // through, as does a row whose scores grew.
      {
        const float rs = exps(std::bool_constant<!kSeed>{}, shift, pen[qb]);
        if (__ballot(!(rs <= kSumLimit)) == 0) {
          l_run[qb] += rs;
          return 1.f;
        }
      }
      // Exact path: the row max of sacc (max chains, then the exchange between
      // the lane halves, and with 16 x 16 tiles between the 16-lane rows). The
      // reference moves up to the row max, or,
      // on a row's first unmasked tile, to it from wherever it was.
      float pm[8];
      constexpr int NE = KB * AE;   // the lane's scores of the row (32 either way)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pm[j] = vmax(sacc[(2 * j) / AE][(2 * j) % AE], sacc[(2 * j + 1) / AE][(2 * j + 1) % AE]);
#pragma unroll
      for (int e = 16; e < NE; e += 2)
        pm[(e / 2) % 8] = vmax(pm[(e / 2) % 8], vmax(sacc[e / AE][e % AE], sacc[(e + 1) / AE][(e + 1) % AE]));
      float mx = vmax(vmax(vmax(pm[0], pm[1]), vmax(pm[2], pm[3])),
                      vmax(vmax(pm[4], pm[5]), vmax(pm[6], pm[7])));
      mx = (M16 ? quarters_max(mx) : halves_max(mx)) - shift;   // row max of u - r
      const bool seen = pen[qb] == 0.f;
      // d: how far the reference moves (0 while a row has no unmasked key)
      const float d = seen ? vmax(mx, 0.f) : (mx == -INFINITY ? 0.f : mx);
      // O and l are still 0 on an unseen row: no rescale
      const float alpha = (!seen || d == 0.f) ? 1.f : __builtin_amdgcn_exp2f(-d);
      r_ref[qb] += d;
      if constexpr (kKeepSeed) {
#pragma unroll
        for (int i = 0; i < AE; ++i) neg_r[qb][i] = -r_ref[qb];
      }
      if (mx != -INFINITY) pen[qb] = 0.f;
      const float rs = exps(std::true_type{}, shift + d, 0.f);
      l_run[qb] = l_run[qb] * alpha + rs;
      return alpha;
    };
    auto rescale = [&](int qb, float alpha) __attribute__((always_inline)) {
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int i = 0; i < AE; ++i) oacc[qb][b][i] *= alpha;
      }
    };

    if constexpr (W == 8) {
    // ---- ping-pong tile loop ----------------------------------------------------
    // Half-step h: group 0 runs its MFMA phase for tile h/2 when h is even and
    // the softmax of tile h/2 when h is odd; group 1 lags by one half-step.
    // Each wave issues its share of K(s+1) at the start of half-step 2s and of
    // V(s) at the start of half-step 2s+1 (spreading the load issue, which
    // stalls the issuing wave), and waits for both at the end of 2s+1. One
    // workgroup barrier per tile, after odd half-steps, is enough: every
    // buffer a load overwrites was last read in half-step 2s-1 or earlier.
    // Between barriers the two groups keep their phase offset by themselves,
    // since the MFMA and softmax phases take about as long. The loop is
    // unrolled by four half-steps so that every access names one fixed LDS
    // buffer.
    const int grp_id = wave / kGroupWaves;
    Acc sacc[QB][KB];
    auto mfma_phase = [&](int t, const u32x4* kb, const u32x4* vb) __attribute__((always_inline)) {
      // One instruction stream for every tile up to my_total: at t = 0 the
      // PV half multiplies the zeroed P by the zeroed V buffer (a no-op), and at
      // t = my_total the QK half computes a score tile nobody reads. A
      // branch per product costs more (registers at the join) than these
      // 32 MFMAs per pass.
      if (t <= my_total) {
        __builtin_amdgcn_s_setprio(1);
        pvqk(sacc, kb, vb, kOn{}, kOn{});
        __builtin_amdgcn_s_setprio(0);
      }
    };
    auto valu_phase = [&](int t) __attribute__((always_inline)) {
      if (t >= 0 && t < my_total) {
        const bool masked = t >= my_full;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          bf16x8 pnew[PS];
          const float alpha = softmax(sacc[qb], qb, tile_of(t), masked, pnew);
          rescale(qb, alpha);
#pragma unroll
          for (int ps = 0; ps < PS; ++ps) pprev[qb][ps] = pnew[ps];
        }
      }
    };
    const int h_end = 2 * ntiles + 1;  // last half-step (group 1's final PV)
    // One half-step of group G (compile time): this wave's share of one tile
    // load, then the group's phase, then (odd half-steps) the wait for the
    // loads and the workgroup barrier. Both groups run the same sequence of
    // barriers, each from its own copy of the loop.
    auto half_step = [&](auto g_c, auto hp, int h) __attribute__((always_inline)) {
      constexpr int G = decltype(g_c)::value;
      constexpr int HP = decltype(hp)::value;   // h mod 4
      constexpr int SP = (HP >> 1) & 1;         // parity of s = h / 2
      constexpr bool EVEN = (HP & 1) == 0;
      u32x4* kc = SP ? kbuf1 : kbuf0;           // K(s)
      u32x4* kn = SP ? kbuf0 : kbuf1;           // K(s+1)
      u32x4* vp = SP ? vbuf0 : vbuf1;           // V(s-1)
      u32x4* vc = SP ? vbuf1 : vbuf0;           // V(s)
      const int s2 = h >> 1;
      if (EVEN) {
        if (s2 + 1 < ntiles) load_k(kn, tile_of(s2 + 1));
      } else {
        if (s2 < ntiles) load_v(vc, tile_of(s2));
      }
      if (active) {
        if (EVEN == (G == 0)) mfma_phase(s2, kc, vp);
        else valu_phase(G == 0 ? s2 : s2 - 1);
      }
      if (!EVEN) {
        wait_vm();
        __syncthreads();
      }
    };
    auto run_group = [&](auto g_c) __attribute__((always_inline)) {
      for (int h = 0; h <= h_end; h += 4) {
        half_step(g_c, std::integral_constant<int, 0>{}, h);
        half_step(g_c, std::integral_constant<int, 1>{}, h + 1);
        if (h + 2 > h_end) break;
        half_step(g_c, std::integral_constant<int, 2>{}, h + 2);
        half_step(g_c, std::integral_constant<int, 3>{}, h + 3);
      }
    };
    // K(0), and zeros in the V buffer the first (empty) PV half reads: it
    // multiplies the zeroed P by them, and V data there (0 * Inf = NaN for a
    // key some rows never see) could change those rows.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) pprev[qb][ps] = bf16x8{};
    load_k(kbuf0, tile_of(0));
    for (int i = tid; i < TL::VCHUNKS + TL::VSLACK; i += kWaves * 64) vbuf1[i] = u32x4{0u, 0u, 0u, 0u};
    prep_q();
    wait_vm();
    __syncthreads();
    if (grp_id == 0) run_group(std::integral_constant<int, 0>{});
    else run_group(std::integral_constant<int, 1>{});

    } else {
    // ---- software-pipelined tile loop ----------------------------------------
    // Iteration t runs the MFMA stream O += P(t-1) V(t-1), S(t) = K(t) Q^T,
    // then the softmax of S(t), while K(t+1) and V(t) stream into the other
    // buffers; the two workgroups on a SIMD pair overlap each other's MFMA
    // and softmax work. Every wave runs iterations 0 .. ntiles (the loads and
    // the barrier are shared); a wave with n tiles of its own computes
    // S(0) alone at t = 0, both products for t < n, the last PV product
    // alone at t = n, and nothing after that. The loop is unrolled by two so
    // every access names one fixed LDS buffer.
    Acc sacc[QB][KB];
    // modes: 0 loads and barrier only, 1 first tile (QK), 2 both products, 3 last PV
    auto iteration = [&](auto parity, auto mode, int t) __attribute__((always_inline)) {
      constexpr int PAR = decltype(parity)::value;
      constexpr int MODE = decltype(mode)::value;
      u32x4* kcur = PAR ? kbuf1 : kbuf0;
      u32x4* knext = PAR ? kbuf0 : kbuf1;
      u32x4* vprev = PAR ? vbuf0 : vbuf1;
      u32x4* vcur = PAR ? vbuf1 : vbuf0;
      if (t > 0) {   // the prologue issued iteration 0's loads
        if (t + 1 < ntiles) load_k(knext, tile_of(t + 1));
        if (t < ntiles) load_v(vcur, tile_of(t));
      }
      if constexpr (MODE != 0) {
        // Priority for the MFMA stream at d = 64 only: measured with two
        // workgroups per SIMD pair, it helps d = 64 and slows d = 128 (the
        // broadcast workload) by a few percent.
        if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
        pvqk(sacc, kcur, vprev, std::bool_constant<MODE != 1>{}, std::bool_constant<MODE != 3>{});
        if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
        if constexpr (MODE != 3) {
          const bool masked = t >= my_full;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            bf16x8 pnew[PS];
            const float alpha = softmax(sacc[qb], qb, tile_of(t), masked, pnew);
            rescale(qb, alpha);
#pragma unroll
            for (int ps = 0; ps < PS; ++ps) pprev[qb][ps] = pnew[ps];
          }
        }
      }
      wait_vm();
      __syncthreads();
    };
    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;
    using Idle = std::integral_constant<int, 0>;
    using First = std::integral_constant<int, 1>;
    using Both = std::integral_constant<int, 2>;
    using Last = std::integral_constant<int, 3>;
    // The prologue issues K(0) and iteration 0's loads, V(0) and K(1), right
    // behind the queries', so that their round trips overlap. It waits for
    // the queries and K(0) only: V(0) and K(1), issued last, may still be in
    // flight (every wave issues at least VLOADS / W and KLOADS / W of them),
    // and iteration 0 waits for them.
    load_k(kbuf0, tile_of(0));
    load_v(vbuf0, tile_of(0));
    if (1 < ntiles) load_k(kbuf1, tile_of(1));
    prep_q();
    if (1 < ntiles) wait_vm_n<TL::VLOADS / W + TL::KLOADS / W>();
    else wait_vm_n<TL::VLOADS / W>();
    __syncthreads();
    int t = 0;
    const int n = active ? my_total : 0;   // tiles this wave computes
    if (n > 0) {
      iteration(Even{}, First{}, 0);
      for (t = 1; t + 1 < n; t += 2) {
        iteration(Odd{}, Both{}, t);
        iteration(Even{}, Both{}, t + 1);
      }
      if (t < n) iteration(Odd{}, Both{}, t++);
      if (t & 1) iteration(Odd{}, Last{}, t);
      else iteration(Even{}, Last{}, t);
      ++t;
    }
    for (; t <= ntiles; ++t) {
      if (t & 1) iteration(Odd{}, Idle{}, t);
      else iteration(Even{}, Idle{}, t);
    }

    }

    // ---- epilogue: O = O^T / l, round to bf16, store ---------------------------
    // Lanes l and l + 32 hold the same row: lane l columns 8m .. 8m+3 of each
    // group m of a 32-column block, lane l + 32 columns 8m+4 .. 8m+7. One
    // lane-half swap per pair of groups (2q, 2q+1) gives lane l the eight
    // columns of group 2q and lane l + 32 those of group 2q+1: half as many
    // stores, 16 bytes each. The swap runs in every lane; only the stores
    // depend on the row.
    if (active && M16) {
      // 16 x 16 tiles: lane l holds d = 16 b + 4 (l / 16) + 0..3 of query
      // row0 + 16 qb + l % 16, so 16-lane rows 2j and 2j + 1 hold the two
      // halves of columns 16 b + 8 j .. + 7. One row-pair swap per pair of d
      // blocks (2m, 2m + 1) gives the even row those eight columns of block 2m
      // and the odd row those of block 2m + 1: 16-byte stores.
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float l = quarters_sum(l_run[qb]);
        const float inv = (l > 0.f) ? 1.f / l : 0.f;
        const int row = me.row0 + QR * qb + qcol;
        __bf16* orow = og + (size_t)row * q_rs;
#pragma unroll
        for (int m = 0; m < DB / 2; ++m) {
          uint32_t w[2][2];
#pragma unroll
          for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const bf16x2 h = {(__bf16)(oacc[qb][2 * m + k][2 * e] * inv),
                                (__bf16)(oacc[qb][2 * m + k][2 * e + 1] * inv)};
              w[k][e] = __builtin_bit_cast(uint32_t, h);
            }
          const auto s0 = __builtin_amdgcn_permlane16_swap(w[0][0], w[1][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane16_swap(w[0][1], w[1][1], false, false);
          const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
          const int b = 2 * m + (qgrp & 1);
          if (row < me.lq) *(u32x4*)(orow + b * 16 + 8 * (qgrp >> 1)) = v;
        }
      }
    } else if (active) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float l = halves_sum(l_run[qb]);
        const float inv = (l > 0.f) ? 1.f / l : 0.f;
        const int row = me.row0 + 32 * qb + col;
        __bf16* orow = og + (size_t)row * q_rs;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bf16x2 h = {(__bf16)(oacc[qb][b][8 * q + 2 * e] * inv),
                                (__bf16)(oacc[qb][b][8 * q + 2 * e + 1] * inv)};
              w[e] = __builtin_bit_cast(uint32_t, h);
            }
            const auto s0 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
            const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
            if (row < me.lq) *(u32x4*)(orow + b * 32 + 16 * q + 8 * half) = v;
          }
      }
    }
  }
}

// Host-side launcher (one instance per head dim, causal flag and wave count).
hipError_t launch_bf16(const Params& p, int D, bool causal, hipStream_t stream) {
  // An error left pending by an earlier HIP call on this thread is dropped
  // here, so that the status returned after the launch is this launch's.
  (void)hipGetLastError();
  dim3 grid(p.T), block(p.waves * 64);
#define ATTN_LAUNCH(DD, CC, WW)                                                                 \
  do {                                                                                          \
    if (p.q_offsets != nullptr)                                                                 \
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<DD, CC, WW, kJagged>), grid, block, 0, stream, p); \
    else if (p.block_mask != nullptr)                                                           \
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<DD, CC, WW, kSparse>), grid, block, 0, stream, p); \
    else                                                                                        \
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<DD, CC, WW, kDense>), grid, block, 0, stream, p);  \
  } while (0)
  if (p.waves == 8) {
    if (D == 128) {
      if (causal) ATTN_LAUNCH(128, true, 8); else ATTN_LAUNCH(128, false, 8);
    } else {
      if (causal) ATTN_LAUNCH(64, true, 8); else ATTN_LAUNCH(64, false, 8);
    }
  } else {
    if (D == 128) {
      if (causal) ATTN_LAUNCH(128, true, 4); else ATTN_LAUNCH(128, false, 4);
    } else {
      if (causal) ATTN_LAUNCH(64, true, 4); else ATTN_LAUNCH(64, false, 4);
    }
  }
#undef ATTN_LAUNCH
  return hipGetLastError();
}

// Long d=128 key sequences run the 8-wave ping-pong schedule; shorter ones
// (and d=64, whose softmax outweighs its MFMA work) the 4-wave schedule.
constexpr int kPingPongMinKeys = 4096;

// Work decomposition for the bf16 kernel: query rows are split into wave
// blocks of kRowsPerWave; a workgroup takes `waves` consecutive blocks of one
// (batch entry, head), or, for short sequences, whole batch entries of a
// power-of-two number of blocks each (so a workgroup never straddles an entry).
// The environment variable ATTN_BF16_WAVES=4|8 overrides the choice (for
// tuning and for testing both schedules on the same inputs).
static int waves_override() {
  static const int v = [] {
    const char* e = getenv("ATTN_BF16_WAVES");
    if (e != nullptr && (e[0] == '4' || e[0] == '8') && e[1] == '\0') return e[0] - '0';
    return 0;
  }();
  return v;
}

// K/V bytes the units of one causal chunk may span (ATTN_CHUNK_KV_MIB
// overrides, for tuning).
int64_t chunk_kv_bytes() {
  static const int64_t v = [] {
    const char* e = getenv("ATTN_CHUNK_KV_MIB");
    const long m = (e != nullptr) ? strtol(e, nullptr, 10) : 0;
    return (int64_t)(m > 0 ? m : 4) << 20;   // one XCD's L2 (measured best of 1..16 MiB)
  }();
  return v;
}

bool plan_bf16(Params& p, int D, bool causal) {
  // K/V of one (batch, head) are addressed through 32-bit buffer offsets;
  // the last tile may run up to 64 rows past Lk.
  const int64_t kv_row_bytes = (int64_t)(p.q_offsets != nullptr ? p.Hkv : 1) * D * 2;
  if (((int64_t)p.Lk + 64) * kv_row_bytes > 0x7fffffff) return false;
  int W = (D == 128 && p.Lk >= kPingPongMinKeys) ? 8 : 4;
  if (waves_override() != 0) W = waves_override();
  // block-sparse: a workgroup's rows must lie in one query block
  if (p.block_mask != nullptr) {
    if (p.blk % (W * kRowsPerWave) != 0) W = 4;
    if (p.blk % (W * kRowsPerWave) != 0 || p.nKB > kMaxKeyBlocks) return false;
  }
  p.waves = W;
  const int64_t nrb = ((int64_t)p.Lq + kRowsPerWave - 1) / kRowsPerWave;
  if (nrb >= W) {
    p.P = (int)(((nrb + W - 1) / W) * W);
    p.G = 1;
    p.nMT = p.P / W;
    p.NG = p.NB;
  } else {
    int P = 1;
    while (P < nrb) P *= 2;   // whole entries per workgroup
    p.P = P;
    p.G = W / P;
    p.nMT = 1;
    p.NG = (p.NB + p.G - 1) / p.G;
  }
  const int64_t T = (int64_t)p.NG * p.H * p.nMT;
  if (T > 0x7fffffff) return false;
  p.T = (int)T;
  // Keep all tiles that read one K/V head on one XCD (its L2), so each K/V
  // head streams from memory into a single L2. Broadcast tiles of one head
  // are ordered by candidate group; runs of 16 groups usually share a user.
  // Causal dense problems whose K/V heads are too few tiles to fill an XCD
  // share several heads per chunk, ordered longest-first inside it: up to an
  // XCD's share of the units, as long as their K/V (read concurrently) stay
  // within kChunkKVBytes, so that K/V re-reads keep hitting the caches.
  p.units = 1;
  if (causal && p.cand2user == nullptr) {
    const int64_t share = (p.NG * (int64_t)p.Hkv + 7) / 8;
    const int64_t kv_unit = (int64_t)p.Lk * D * 2 * 2;   // K and V of one unit (at most)
    const int64_t fit = kv_unit > 0 ? chunk_kv_bytes() / kv_unit : share;
    p.units = (int)std::max<int64_t>(1, std::min(share, fit));
  }
  p.chunk = (p.cand2user == nullptr) ? p.units * p.nMT * (p.H / p.Hkv) : 16;
  return true;
}

}  // namespace attn
