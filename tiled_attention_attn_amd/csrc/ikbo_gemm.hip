// In-kernel broadcast (IKBO) linear layer for gfx950: bf16 MFMA GEMM with
// fp32 accumulation and a gathered-row epilogue.
//
// Method: "How We Built TLX" (Chinese translation, "Case study 2: in-kernel
// broadcast optimisation for RecSys") speeds up a linear-compression kernel
// by splitting the matrix product, aligning memory and fusing the broadcast:
// a user's features are the same for all of its candidates, so the user half
// of the product is computed once per user and broadcast to the candidates
// inside the kernel instead of being replicated in memory. For a linear layer
// with weight W = [W_user | W_cand] over the concatenated features
// [x_user[cand2user[c]], x_cand[c]], candidate c's output is
//     Y[c] = x_cand[c] W_cand^T + (x_user W_user^T + bias)[cand2user[c]].
// Step 1 writes Z = x_user W_user^T + bias (fp32, one row per user); step 2
// computes x_cand W_cand^T and adds row Z[cand2user[c]] in its epilogue.
//
// Both steps run one kernel: C[M, N] = A[M, K] B[N, K]^T (+ bias or Z[zrow]).
// Operands follow the linear-layer layout (B is [out, in], rows contiguous in
// K), so both MFMA operands read 16 contiguous bytes per lane from LDS. A
// workgroup owns a TM x TN output tile (256 x 256, or a smaller one when that
// grid would leave CUs idle), split over its waves as blocks of
// v_mfma_f32_32x32x16_bf16 computed transposed (C^T = B A^T), so that each
// lane holds one output row and runs of 4 consecutive columns. The wave tile
// sets the LDS reads per MFMA (128 x 64 reads 6 fragments per 8 MFMAs). K
// advances 64 at a time through two LDS stages filled with direct-to-LDS
// buffer loads, each filling one 1 KB LDS window with 8 whole rows of the
// stage; the windows are staggered by one 16-byte chunk so that operand
// reads are free of bank conflicts. On a persistent grid the last two
// stages of a tile load the next tile's first two, so the K loop runs on
// across tiles. With bf16 output, a tile's results wait in registers until
// the next tile's addend loads are issued and are stored behind them, so
// that the stores drain while that tile computes.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "gemm_params.h"

namespace attn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

// Word 3 of a raw buffer descriptor (gfx9 family): 32-bit data format, no
// swizzle; with stride 0 an access is in range iff its offset is below
// num_records, and out-of-range loads return zero.
constexpr int kBufferWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;   // above every num_records used here
constexpr int kSchedMFMA = 0x008, kSchedDSRead = 0x100;

// s_waitcnt vmcnt(0): wait for this wave's direct-to-LDS loads.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): at most N of this wave's vector memory operations (loads
// and stores, which gfx9 counts together and retires in issue order) remain.
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroups are dispatched round-robin over the 8 XCDs (XCD x runs ids x,
// x+8, ...). Give each XCD a contiguous range of tiles, so the column tiles
// of one row block (which share their A rows) run on one XCD's L2.
__device__ __forceinline__ int xcd_tile(int w, int T) {
  const int x = w & 7, i = w >> 3, q = T >> 3, r = T & 7;
  return x * q + (x < r ? x : r) + i;
}

}  // namespace

// Tile configurations (TM x TN per workgroup, waves as WM x WN):
//   0: 256 x 256, 2 x 4 waves of 128 x 64, one workgroup per CU;
//   1: 128 x 128, 2 x 2 waves of 64 x 64, two per CU;
//   2: 128 x 64,  2 x 2 waves of 64 x 32, two per CU (small grids);
//   3: 128 x 64 as 2, one per CU with four LDS stages (grids of at most one
//      tile per CU: one wave per SIMD hides load latency only by loading
//      further ahead).
// All keep the accumulators in architected VGPRs.
template <int CFG>
struct GemmShape {
  static constexpr bool kBig = CFG == 0;
  static constexpr int TM = kBig ? 256 : 128;
  static constexpr int TN = kBig ? 256 : CFG == 1 ? 128 : 64;
  static constexpr int kWavesM = 2, kWavesN = kBig ? 4 : 2;
  static constexpr int kWaves = kWavesM * kWavesN;
  static constexpr int MB = TM / kWavesM / 32;     // 32 x 32 blocks per wave, rows
  static constexpr int NB = TN / kWavesN / 32;     // and columns
  static constexpr int kPerCU = kBig || CFG == 3 ? 1 : 2;
  static constexpr int kStages = CFG == 3 ? 4 : 2;
  static constexpr int BK = 64;                    // K per LDS stage
  // Workgroups per CU for the register budget: 3 runs one (its LDS allows no
  // more) but takes the budget of two, 256 registers per wave. With the whole
  // file the compiler moves the accumulators to AGPRs and copies each addend
  // load into them behind its own wait.
  static constexpr int kRegsPerCU = kBig ? 1 : 2;
};

template <int CFG, bool GATHER, bool OUT_F32>
__global__ __launch_bounds__(GemmShape<CFG>::kWaves * 64, GemmShape<CFG>::kRegsPerCU) void
ikbo_gemm_kernel(const GemmParams p) {
  using S = GemmShape<CFG>;
  constexpr int kWaves = S::kWaves, MB = S::MB, NB = S::NB, TM = S::TM, TN = S::TN;
  constexpr int WTM = MB * 32, WTN = NB * 32;     // wave tile
  constexpr int kBK = S::BK;                      // K per LDS stage
  constexpr int kRowChunks = kBK / 8;             // 16-byte chunks of one row in a stage
  constexpr int kSub = kBK / 16;                  // MFMA k-substeps per stage
  static_assert(kSub % 2 == 0, "substeps alternate between two fragment slots");
  // Stage layout: wave load n fills window n, 1 KB holding rows n, n + NW,
  // n + 2 NW, ... (NW = rows / 8 windows) row-major; windows start kWin = 65
  // chunks apart. Row r, column chunk c is at chunk
  // (r % NW) * kWin + (r / NW) * kRowChunks + c. An operand read has 16 lanes
  // on 16 consecutive rows at one chunk: the one-chunk stagger of the windows
  // (and the 128-byte row offset inside a window) puts them on distinct
  // 16-byte bank groups, and every load reads whole rows with no idle lane.
  static_assert(kRowChunks == 8, "eight rows per 1 KB window");
  constexpr int kWin = 65;
  constexpr int kNWA = TM / 8, kNWB = TN / 8;     // windows (= wave loads) per stage
  static_assert(32 % kNWA == 0 && 32 % kNWB == 0, "row blocks of 32 span whole window rounds");
  constexpr int kChunksA = kNWA * kWin, kChunksB = kNWB * kWin;   // chunks per stage
  constexpr int kLoadsA = kNWA, kLoadsB = kNWB;                   // wave-wide loads
  constexpr int kPerA = (kLoadsA + kWaves - 1) / kWaves;
  constexpr int kPerB = (kLoadsB + kWaves - 1) / kWaves;
  // Separate arrays per stage buffer: the compiler then knows that reads of
  // one buffer do not wait for direct-to-LDS loads still landing in another.
  constexpr int kRingA = S::kStages > 2 ? kChunksA : 1, kRingB = S::kStages > 2 ? kChunksB : 1;
  __shared__ u32x4 abuf0[kChunksA];
  __shared__ u32x4 abuf1[kChunksA];
  __shared__ u32x4 abuf2[kRingA];
  __shared__ u32x4 abuf3[kRingA];
  __shared__ u32x4 bbuf0[kChunksB];
  __shared__ u32x4 bbuf1[kChunksB];
  __shared__ u32x4 bbuf2[kRingB];
  __shared__ u32x4 bbuf3[kRingB];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / S::kWavesN, wn = wave % S::kWavesN;
  // Persistent grid: a workgroup runs tiles blockIdx.x, +G, +2G, ... (G =
  // gridDim.x, a multiple of 8 whenever it is below the tile count, so the
  // workgroup stays on one XCD).
  // bf16 output with two stages: a whole tile's results wait in registers
  // (converted and lane-swapped) until the next tile's addend loads (and its
  // first two stages', unless the previous tile loaded them) are issued; its
  // stores follow them and drain under that tile's first two stages. Edge tiles (rows past M or columns past N), and
  // the four-stage configuration (picked for grids of one round), store at
  // once. gfx9 counts loads and stores in one counter (vmcnt) and retires
  // them in issue order, so a wave waits for a stage with a count that leaves
  // the later stores outstanding; every store is therefore issued, whatever
  // the tile.
  // When A and B each leave half the waves one load short, B's loads start
  // half a workgroup later, so every wave issues the same number per stage
  // and the counted waits below are exact.
  constexpr int kRotB =
      (kLoadsA % kWaves == kWaves / 2 && kLoadsB % kWaves == kWaves / 2) ? kWaves / 2 : 0;
  constexpr int kMinLoads = kRotB ? (kLoadsA + kLoadsB) / kWaves   // per wave and stage
                                  : kLoadsA / kWaves + kLoadsB / kWaves;
  constexpr int kStores = MB * NB * 2;                            // 16-byte stores per wave
  constexpr bool kPend = !OUT_F32 && S::kStages == 2;
  u32x4 pend[MB][NB][2];
  int pm0 = -1, pn0 = 0;
  const uint32_t crow = (uint32_t)p.N * 2;
  // One offset per lane: row wm*WTM + col, column wn*WTN + 8*half of the
  // tile; block row i goes in the scalar offset, the column block in the
  // instruction's immediate. With nothing pending (pm0 < 0) the range is
  // empty and the stores are dropped.
  auto store_pending = [&](int col, int half) __attribute__((always_inline)) {
    const uint32_t svoff = (uint32_t)(wm * WTM + col) * crow + (uint32_t)(wn * WTN + 8 * half) * 2;
    const bool any = pm0 >= 0;
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((char*)p.c + (any ? (size_t)pm0 * crow + (size_t)pn0 * 2 : 0)), (short)0,
        any ? (int)((uint32_t)TM * crow) : 0, kBufferWord3);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          __builtin_amdgcn_raw_buffer_store_b128(pend[i][j][q], crs, svoff + (j * 32 + 16 * q) * 2,
                                                 (int)((uint32_t)(i * 32) * crow), 0);
  };
  // Row block and column tile of the tile a workgroup runs at its step wl.
  auto coords = [&](int wl, int& m0, int& n0) __attribute__((always_inline)) {
    const int tile = xcd_tile(wl, p.tiles);
    int rb, cb;
    if constexpr (CFG == 3) {
      // Column groups of 8 tiles, row blocks inside a group: an XCD's share of
      // the tile order then spans fewer columns of B. On the user half of the
      // broadcast layer (16 x 16 tiles) an XCD's 32 tiles read 4 row blocks of
      // A and 8 column tiles of B, 2 + 2 MB, instead of 1 + 4.2 MB, within its
      // 4 MB L2.
      constexpr int kGW = 8;
      const int nrb = p.tiles / p.tiles_n;
      const int grp = tile / (kGW * nrb);
      const int gcols = min(kGW, p.tiles_n - grp * kGW);
      const int r = tile - grp * kGW * nrb;
      rb = r / gcols;
      cb = grp * kGW + r % gcols;
    } else {
      rb = tile / p.tiles_n;
      cb = tile % p.tiles_n;
    }
    m0 = rb * TM;
    n0 = cb * TN;
  };
  // Buffer descriptors start at the tile's first row and end with the last
  // valid row's K-th element: chunks of rows past M (or N) read as zero.
  const uint32_t a_row = (uint32_t)p.lda * 2, b_row = (uint32_t)p.ldb * 2;
  auto a_rsrc = [&](int m0) __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)p.a + (size_t)m0 * a_row), (short)0,
        (int)((uint32_t)(p.M - m0 - 1) * a_row + (uint32_t)p.K * 2), kBufferWord3);
  };
  auto b_rsrc = [&](int n0) __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)p.b + (size_t)n0 * b_row), (short)0,
        (int)((uint32_t)(p.N - n0 - 1) * b_row + (uint32_t)p.K * 2), kBufferWord3);
  };
  const int nst = (p.K + kBK - 1) / kBK;
  // Persistent two-stage ring with an even number of stages: the last two
  // steps of a tile load the next tile's first two stages into the buffers
  // they free, so that a tile starts with its operands in LDS; its gathered
  // row indices come with its stage 0. The LDS buffers then alternate across
  // tiles as they do inside one.
  const bool xpre = kPend && nst >= 2 && (nst & 1) == 0;
  // Gathered row indices go through LDS: each wave loads the zrow entries of
  // its own WTM rows (consecutive) into a slot of its own with direct-to-LDS
  // loads, and reads its lanes' entries from there. Loaded one tile ahead,
  // they then never hold up a register a tile's early code might touch.
  constexpr int kZLoads = WTM / 64;   // 4-byte loads per wave and tile
  static_assert(WTM % 64 == 0, "row slots are whole wave loads");
  __shared__ int zslot[GATHER ? kWaves * WTM : 1];
  auto load_zrow = [&](int m0t) __attribute__((always_inline)) {
    const int r0 = m0t + wm * WTM;
    const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.zrow + r0), (short)0, max(p.M - r0, 0) * 4, kBufferWord3);
#pragma unroll
    for (int k = 0; k < kZLoads; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          zrs, (void LDS_AS*)(zslot + wave * WTM + k * 64), 4,
          (uint32_t)(k * 64 + (threadIdx.x & 63)) * 4, 0, 0, 0);
  };
  if (GATHER && (int)blockIdx.x < p.tiles) {
    int m0f, n0f;
    coords(blockIdx.x, m0f, n0f);
    load_zrow(m0f);
    wait_vm();
  }
  for (int wl = blockIdx.x; wl < p.tiles; wl += gridDim.x) {
  const bool first = wl == (int)blockIdx.x;
  const bool pre = xpre && !first;                 // stages 0 and 1 already loaded
  const bool has_next = wl + (int)gridDim.x < p.tiles;
  const bool load_next = xpre && has_next;        // this tile loads the next one's
  // Per-lane indices are recomputed every tile (the empty asm hides that
  // they are loop-invariant): hoisted out of the tile loop they would stay
  // live across the tile boundary, where the pending output needs the room.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int half = lane >> 5, col = lane & 31;
  int m0, n0, m0n = 0, n0n = 0;
  coords(wl, m0, n0);
  if (has_next) coords(wl + (int)gridDim.x, m0n, n0n);
  const __amdgpu_buffer_rsrc_t arsrc = a_rsrc(m0), brsrc = b_rsrc(n0);
  const __amdgpu_buffer_rsrc_t arsrc_n = a_rsrc(m0n), brsrc_n = b_rsrc(n0n);

  // Wave load n fills window n of a stage: lane i takes row n + NW * (i / 8),
  // column chunk i % 8.
  const int wave_b = (wave + kRotB) % kWaves;
  const uint32_t lrow = (uint32_t)lane / kRowChunks, lchunk = (uint32_t)lane % kRowChunks;
  uint32_t aoff[kPerA], boff[kPerB];
#pragma unroll
  for (int j = 0; j < kPerA; ++j)
    aoff[j] = ((uint32_t)(wave + j * kWaves) + lrow * kNWA) * a_row + lchunk * 16;
#pragma unroll
  for (int j = 0; j < kPerB; ++j)
    boff[j] = ((uint32_t)(wave_b + j * kWaves) + lrow * kNWB) * b_row + lchunk * 16;
  // Stage s covers K columns 64s .. 64s+63; in a last stage cut by K, the
  // chunks past K take the out-of-range offset too.
  // (Offsets are passed as plain uint32_t values: in this template an
  // array-element argument made the host pass drop the kernel's stub.)
  auto load_stage_from = [&](__amdgpu_buffer_rsrc_t ars, __amdgpu_buffer_rsrc_t brs, u32x4* adst,
                             u32x4* bdst, int s) __attribute__((always_inline)) {
    const uint32_t koff = (uint32_t)s * (kBK * 2);
    const bool ragged = p.K - s * kBK < kBK;                  // chunks past K in this stage
    const int lim = min((p.K - s * kBK) >> 3, kRowChunks);   // valid column chunks
#pragma unroll
    for (int j = 0; j < kPerA; ++j) {
      const int n = wave + j * kWaves;
      if (j < kPerA - 1 || n < kLoadsA) {
        uint32_t o = aoff[j] + koff;
        if (ragged && (int)lchunk >= lim) o = kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (void LDS_AS*)(adst + n * kWin), 16,
                                                 (uint32_t)o, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < kPerB; ++j) {
      const int n = wave_b + j * kWaves;
      if (j < kPerB - 1 || n < kLoadsB) {
        uint32_t o = boff[j] + koff;
        if (ragged && (int)lchunk >= lim) o = kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (void LDS_AS*)(bdst + n * kWin), 16,
                                                 (uint32_t)o, 0, 0, 0);
      }
    }
  };
  auto load_stage = [&](u32x4* adst, u32x4* bdst, int s) __attribute__((always_inline)) {
    load_stage_from(arsrc, brsrc, adst, bdst, s);
  };

  // acc[i][j]: rows m0 + wm*WTM + i*32 .. +31 (one per lane) by columns
  // n0 + wn*WTN + j*32 .. +31 (in registers): register 4g + e holds column
  // j*32 + 8g + 4*half + e of the wave's block (the MFMA output row index).
  // The accumulators start from the row's addend (row zrow[m] of Z, or the
  // bias), so the products are summed onto it and the epilogue only stores.
  // Every lane issues the same loads whatever its row and columns (rows past
  // M and columns past N, which are never stored, read a valid row and the
  // last run of 4 columns), so that a wave's count of memory operations is
  // fixed. With its first stages already in LDS, a tile does not wait for
  // these loads before it starts: each MFMA waits only for its own
  // accumulator. A row whose zrow is out of range gets NaN in the epilogue.
  // N is a multiple of 4: each run of 4 columns is wholly inside or outside.
  // A tile whose first two stages the previous one loaded waits here for its
  // stage 0: what may still be in flight is stage 1's loads (at least
  // kMinLoads per wave), issued after them.
  if (pre) wait_vm_n<kMinLoads>();
  // Without that, a tile after the first loads its row indices now.
  if (GATHER && !xpre && !first) {
    load_zrow(m0);
    wait_vm();
  }
  asm volatile("" ::: "memory");   // the row-index reads stay after these waits
  f32x16 acc[MB][NB];
  uint32_t badm = 0;   // bit i: row block i's zrow is out of range
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const float* src = p.bias;
    if constexpr (GATHER) {
      const int zr = zslot[wave * WTM + i * 32 + col];
      const bool bad = zr < 0 || zr >= p.Mz;
      badm |= (uint32_t)bad << i;
      src = p.z + (size_t)(bad ? 0 : zr) * p.N;
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = min(n0 + wn * WTN + j * 32 + 8 * g + 4 * half, p.N - 4);
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (GATHER || src != nullptr) v = *(const f32x4*)(src + n);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][4 * g + e] = v[e];
      }
  }
  if constexpr (S::kStages > 2) {
    // Keep the accumulators in VGPRs: in AGPRs, every addend load above is
    // copied over behind a wait of its own.
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) asm volatile("" : "+v"(acc[i][j]));
  }

  // Fragments of one k-substep (16 of K): MB of A and NB of B, two slots.
  bf16x8 av[2][MB], bv[2][NB];
  auto read = [&](const u32x4* ab, const u32x4* bb, int s, int slot)
                  __attribute__((always_inline)) {
    // row wm*WTM + i*32 + col: window col % NW, row (wm*WTM + i*32) / NW +
    // col / NW inside it (NW divides 32)
    const int abase = (col % kNWA) * kWin + (col / kNWA) * kRowChunks + half;
    const int bbase = (col % kNWB) * kWin + (col / kNWB) * kRowChunks + half;
#pragma unroll
    for (int i = 0; i < MB; ++i)
      av[slot][i] = __builtin_bit_cast(
          bf16x8, ab[abase + ((wm * WTM + i * 32) / kNWA) * kRowChunks + 2 * s]);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      bv[slot][j] = __builtin_bit_cast(
          bf16x8, bb[bbase + ((wn * WTN + j * 32) / kNWB) * kRowChunks + 2 * s]);
  };
  auto mfma = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[slot][j], av[slot][i], acc[i][j],
                                                            0, 0, 0);
  };
  // Reads of the next substep interleaved with the MFMAs of this one.
  auto interleave = [&]() __attribute__((always_inline)) {
    constexpr int R = MB + NB, Q = MB * NB / R, E = MB * NB % R;
#pragma unroll
    for (int r = 0; r < E; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, Q + 1, 0);
    }
#pragma unroll
    for (int r = E; r < R; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
      if constexpr (Q > 0) __builtin_amdgcn_sched_group_barrier(kSchedMFMA, Q, 0);
    }
  };
  // One stage from buffer (ab, bb) whose substep 0 is already in slot 0:
  // substeps 0 .. kSub-2 here, each with the next one's reads; the last
  // substep's MFMAs (slot 1) are left to after the barrier.
  auto stage = [&](const u32x4* ab, const u32x4* bb) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 1; s < kSub; ++s) {
      read(ab, bb, s, s & 1);
      mfma((s - 1) & 1);
      interleave();
    }
  };

  // Workgroup barrier without __syncthreads()'s release fence, which would
  // wait for the pending stores too. Each wave has waited (vmcnt) for its own
  // loads of the stage about to be read and waits here for its LDS reads
  // (lgkmcnt); the empty asm statements keep the compiler from moving memory
  // accesses across the barrier.
  auto lds_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unchanged
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  if constexpr (S::kStages == 2) {
    if (!pre) {
      if (nst > 0) load_stage(abuf0, bbuf0, 0);
      if (nst > 1) load_stage(abuf1, bbuf1, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kPend) store_pending(col, half);   // the previous tile's, after the loads
    __builtin_amdgcn_sched_barrier(0);
    // Wait for the addend and stage 0: what may remain is stage 1's loads (at
    // least kMinLoads per wave) and the pending stores (kStores). A tile whose
    // stage 0 the previous one loaded has waited for it already.
    if constexpr (kPend) {
      if (pre) {
      } else if (nst > 1) {
        wait_vm_n<kMinLoads + kStores>();
      } else {
        wait_vm_n<kStores>();
      }
    } else {
      if (nst > 1) wait_vm_n<kMinLoads>(); else wait_vm();
    }
    lds_barrier();
    if (nst > 0) read(abuf0, bbuf0, 0, 0);
    // At the barrier that ends stage t every wave has finished reading buffer
    // t % 2 (the barrier waits for LDS reads) and stage t + 1 has landed; the
    // loads of stage t + 2 then go into buffer t % 2, and substep 3 of stage t
    // runs while substep 0 of stage t + 1 is read (past the last stage that
    // read is of unused data). Stages go in pairs so that every LDS access
    // names one buffer; an odd last stage runs after the loop.
    auto step = [&](u32x4* ab, u32x4* bb, u32x4* nab, u32x4* nbb, int t)
                    __attribute__((always_inline)) {
      stage(ab, bb);
      __builtin_amdgcn_sched_barrier(0);   // keep substep 3's MFMAs after the barrier
      if (kPend && t == 0) wait_vm_n<kStores>(); else wait_vm();
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (t + 2 < nst) load_stage(ab, bb, t + 2);
      else if (load_next) {
        load_stage_from(arsrc_n, brsrc_n, ab, bb, t + 2 - nst);
        if (GATHER && t + 2 == nst) load_zrow(m0n);   // with stage 0, before stage 1
      }
      read(nab, nbb, 0, 0);
      mfma(1);
    };
    int t = 0;
    for (; t + 1 < nst; t += 2) {
      step(abuf0, bbuf0, abuf1, bbuf1, t);
      step(abuf1, bbuf1, abuf0, bbuf0, t + 1);
    }
    if (t < nst) {
      stage(abuf0, bbuf0);
      mfma(1);
    }
  } else {
    // Four stages: stage t lives in buffer t % 4 and loads run three stages
    // ahead. A wave waits only for its own loads of the next stage; the ones
    // it issued after them (up to two stages, at least kMinLoads each) stay
    // in flight.
    auto wait_stage = [&](int after) __attribute__((always_inline)) {
      if (after >= 3) wait_vm_n<3 * kMinLoads>();
      else if (after == 2) wait_vm_n<2 * kMinLoads>();
      else if (after == 1) wait_vm_n<kMinLoads>();
      else wait_vm();
    };
    if (nst > 0) load_stage(abuf0, bbuf0, 0);
    if (nst > 1) load_stage(abuf1, bbuf1, 1);
    if (nst > 2) load_stage(abuf2, bbuf2, 2);
    if (nst > 3) load_stage(abuf3, bbuf3, 3);
    if (nst > 0) {
      wait_stage(min(nst - 1, 3));
      lds_barrier();
      read(abuf0, bbuf0, 0, 0);
    }
    // At the barrier that ends stage t every wave has finished reading buffer
    // t % 4 and stage t + 1 has landed; the loads of stage t + 4 then go into
    // buffer t % 4. The stages issued by then end at min(t + 3, nst - 1).
    auto step = [&](u32x4* ab, u32x4* bb, u32x4* nab, u32x4* nbb, int t)
                    __attribute__((always_inline)) {
      stage(ab, bb);
      __builtin_amdgcn_sched_barrier(0);   // keep substep 3's MFMAs after the barrier
      wait_stage(min(t + 3, nst - 1) - (t + 1));
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (t + 4 < nst) load_stage(ab, bb, t + 4);
      read(nab, nbb, 0, 0);
      mfma(1);
    };
    int t = 0;
    for (; t + 3 < nst; t += 4) {
      step(abuf0, bbuf0, abuf1, bbuf1, t);
      step(abuf1, bbuf1, abuf2, bbuf2, t + 1);
      step(abuf2, bbuf2, abuf3, bbuf3, t + 2);
      step(abuf3, bbuf3, abuf0, bbuf0, t + 3);
    }
    if (t < nst) step(abuf0, bbuf0, abuf1, bbuf1, t);
    if (t + 1 < nst) step(abuf1, bbuf1, abuf2, bbuf2, t + 1);
    if (t + 2 < nst) step(abuf2, bbuf2, abuf3, bbuf3, t + 2);
  }

  if constexpr (GATHER) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
      if ((badm >> i) & 1u)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = __builtin_nanf("");
  }
  // Epilogue. fp32 output: store the accumulators (rows past M and column
  // runs past N are skipped). bf16 output: convert them into the pending
  // registers.
  if constexpr (OUT_F32) {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int m = m0 + wm * WTM + i * 32 + col;
      if (m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WTN + j * 32 + 8 * g + 4 * half;
          if (n >= p.N) continue;
          const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                           acc[i][j][4 * g + 3]};
          *(f32x4*)((float*)p.c + (size_t)m * p.N + n) = v;
        }
    }
  } else {
    // Lanes l and l + 32 hold the same row: lane l columns 8g .. 8g+3 of
    // each group g, lane l + 32 columns 8g+4 .. 8g+7. One lane-half swap per
    // pair of groups (2q, 2q+1) gives lane l all eight columns of group 2q
    // and lane l + 32 those of group 2q+1, for 16-byte stores.
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 h = {(__bf16)acc[i][j][8 * q + 2 * e], (__bf16)acc[i][j][8 * q + 2 * e + 1]};
            w[e] = __builtin_bit_cast(uint32_t, h);
          }
          const auto s0 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
          pend[i][j][q] = u32x4{s0[0], s1[0], s0[1], s1[1]};
        }
    if (kPend && m0 + TM <= p.M && n0 + TN <= p.N) {
      pm0 = m0;
      pn0 = n0;
    } else {
      pm0 = -1;
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int m = m0 + wm * WTM + i * 32 + col;
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int n = n0 + wn * WTN + j * 32 + 8 * (2 * q + half);
            if (m < p.M && n < p.N) {
              __bf16* dst = (__bf16*)p.c + (size_t)m * p.N + n;
              if (n + 8 <= p.N) {
                *(u32x4*)dst = pend[i][j][q];
              } else {
                const u32x2 v = {pend[i][j][q][0], pend[i][j][q][1]};
                *(u32x2*)dst = v;
              }
            }
          }
      }
    }
  }
  // Every wave is done with the LDS stages before the next tile loads into
  // them; stores issued above need not have completed. A next tile whose
  // first stages are already loaded writes LDS only after its first barrier.
  if (!load_next) lds_barrier();
  }
  if constexpr (kPend) store_pending(threadIdx.x & 31, (threadIdx.x >> 5) & 1);
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cached[dev] = n;
  }
  return cached[dev];
}

// One workgroup per slot (kPerCU per CU) when there are more tiles than
// slots; ATTN_GEMM_PERSIST=0 (read once) launches one workgroup per tile.
template <int CFG>
hipError_t launch_cfg(const GemmParams& q, bool gather, bool out_f32, hipStream_t stream) {
  static const bool persist = [] {
    const char* e = getenv("ATTN_GEMM_PERSIST");
    return !(e != nullptr && e[0] == '0');
  }();
  int nblk = q.tiles;
  const int slots = (device_cus() * GemmShape<CFG>::kPerCU) & ~7;
  if (persist && slots >= 8 && q.tiles > slots) nblk = slots;
  const dim3 grid((unsigned)nblk), block(GemmShape<CFG>::kWaves * 64);
  // An error left pending by an earlier HIP call on this thread is dropped
  // here, so that the status returned after the launch is this launch's.
  (void)hipGetLastError();
  if (gather) {
    if (out_f32) hipLaunchKernelGGL((ikbo_gemm_kernel<CFG, true, true>), grid, block, 0, stream, q);
    else hipLaunchKernelGGL((ikbo_gemm_kernel<CFG, true, false>), grid, block, 0, stream, q);
  } else {
    if (out_f32) hipLaunchKernelGGL((ikbo_gemm_kernel<CFG, false, true>), grid, block, 0, stream, q);
    else hipLaunchKernelGGL((ikbo_gemm_kernel<CFG, false, false>), grid, block, 0, stream, q);
  }
  return hipGetLastError();
}

namespace {

int64_t cfg_tiles(int cfg, int64_t M, int64_t N) {
  const int tm = cfg == 0 ? 256 : 128, tn = cfg == 0 ? 256 : cfg == 1 ? 128 : 64;
  return ((M + tm - 1) / tm) * ((N + tn - 1) / tn);
}

// The largest tile that still gives every CU a workgroup (256 CUs), and the
// four-stage configuration when 128 x 64 tiles fit one round at one per CU;
// the environment variable ATTN_GEMM_CFG=0|1|2|3 (read once) forces one.
int pick_cfg(int M, int N) {
  static const int forced = [] {
    const char* e = getenv("ATTN_GEMM_CFG");
    return e ? atoi(e) : -1;
  }();
  if (forced >= 0 && forced <= 3) return forced;
  if (cfg_tiles(0, M, N) >= 256) return 0;
  if (cfg_tiles(1, M, N) >= 256) return 1;
  const int cus = device_cus();
  return cfg_tiles(2, M, N) <= (cus > 0 ? cus : 256) ? 3 : 2;
}

}  // namespace

// Launch one GEMM. A rows beyond what 32-bit buffer offsets reach are handled
// by splitting M into chunks with their own base pointers.
hipError_t launch_ikbo_gemm(GemmParams p, bool gather, bool out_f32, hipStream_t stream) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (!out_f32 && p.N >= (1 << 22)) return hipErrorInvalidValue;   // 32-bit tile offsets
  const int cfg = pick_cfg(p.M, p.N);
  const int tm = cfg == 0 ? 256 : 128, tn = cfg == 0 ? 256 : cfg == 1 ? 128 : 64;
  const int64_t row = (int64_t)p.lda * 2;
  int64_t max_rows = ((int64_t)0x7fffffff - (int64_t)p.K * 2) / (row > 0 ? row : 1) + 1;
  max_rows = max_rows / 256 * 256;
  if (max_rows < 256) return hipErrorInvalidValue;
  p.tiles_n = (p.N + tn - 1) / tn;
  const size_t esz = out_f32 ? 4 : 2;
  for (int64_t m = 0; m < p.M; m += max_rows) {
    GemmParams q = p;
    q.M = (int)(p.M - m < max_rows ? p.M - m : max_rows);
    q.a = (const char*)p.a + m * row;
    q.c = (char*)p.c + (size_t)m * p.N * esz;
    if (gather) q.zrow = p.zrow + m;
    const int64_t tiles = (int64_t)((q.M + tm - 1) / tm) * q.tiles_n;
    if (tiles > 0x7fffffff) return hipErrorInvalidValue;
    q.tiles = (int)tiles;
    const hipError_t err = cfg == 0   ? launch_cfg<0>(q, gather, out_f32, stream)
                           : cfg == 1 ? launch_cfg<1>(q, gather, out_f32, stream)
                           : cfg == 2 ? launch_cfg<2>(q, gather, out_f32, stream)
                                      : launch_cfg<3>(q, gather, out_f32, stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace attn
