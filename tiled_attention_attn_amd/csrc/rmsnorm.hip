// RMS normalisation of bf16 rows for gfx950: the key side of attention on
// normalised queries and keys.
//
// Method: the TLX pages ("How We Built TLX", Chinese translation, the part on
// what explicit layouts make possible) say normalisation can be fused into
// GEMM and attention kernels to save an intermediate memory round trip. The
// attention kernel normalises each query row in registers as it loads it;
// keys are read by every workgroup of their head many times over, so they are
// normalised once here, row by row, into a workspace the attention kernel
// then reads in place of K:
//     y = x / sqrt(mean(x^2) + eps) * gamma      (over the row, fp32, RNE to bf16)
// A row is LPR lanes, 8 elements (16 bytes) each; the sum of squares is
// reduced across those lanes. The kernel reads and writes every byte once.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

}  // namespace

// Each thread handles kRows rows of one lane position; their loads are all
// issued before any arithmetic so that several are in flight per thread.
constexpr int kRows = 4;

template <int LPR>
__global__ __launch_bounds__(kThreads) void rmsnorm_rows_kernel(const __bf16* __restrict__ x,
                                                                __bf16* __restrict__ y,
                                                                const float* __restrict__ gamma,
                                                                float eps, int64_t rows) {
  constexpr int D = 8 * LPR;
  constexpr int kRowsPerPass = kThreads / LPR;     // rows one block covers per pass
  const int part = threadIdx.x % LPR;
  const int64_t row0 = (int64_t)blockIdx.x * (kRowsPerPass * kRows) + threadIdx.x / LPR;
  float g[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) g[e] = gamma != nullptr ? gamma[part * 8 + e] : 1.0f;
  u32x4 raw[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int64_t row = row0 + (int64_t)i * kRowsPerPass;
    raw[i] = u32x4{0u, 0u, 0u, 0u};
    if (row < rows) raw[i] = *(const u32x4*)(x + row * D + part * 8);
  }
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int64_t row = row0 + (int64_t)i * kRowsPerPass;
    const bf16x8 v = __builtin_bit_cast(bf16x8, raw[i]);
    float f[8];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f[e] = (float)v[e];
      ss = __builtin_fmaf(f[e], f[e], ss);
    }
    // The LPR lanes of a row are consecutive and aligned: xor partners stay in it.
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    const float r = 1.0f / sqrtf(ss * (1.0f / D) + eps);
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (__bf16)(f[e] * r * g[e]);
    if (row < rows) *(u32x4*)(y + row * D + part * 8) = __builtin_bit_cast(u32x4, out);
  }
}

// rows x D bf16, contiguous; D in {64, 128}.
hipError_t launch_rmsnorm_rows(const void* x, void* y, const float* gamma, float eps, int64_t rows,
                               int D, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int64_t per_block = (int64_t)(kThreads / (D / 8)) * kRows;
  const int64_t blocks = (rows + per_block - 1) / per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(kThreads);
  // An error left pending by an earlier HIP call on this thread is dropped
  // here, so that the status returned after the launch is this launch's.
  (void)hipGetLastError();
  if (D == 128)
    hipLaunchKernelGGL(rmsnorm_rows_kernel<16>, grid, block, 0, stream, (const __bf16*)x,
                       (__bf16*)y, gamma, eps, rows);
  else if (D == 64)
    hipLaunchKernelGGL(rmsnorm_rows_kernel<8>, grid, block, 0, stream, (const __bf16*)x,
                       (__bf16*)y, gamma, eps, rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace attn
