// Ceiling microbenchmarks for gfx950 (include/attn_ceiling.h): the sustained
// rates of the units the attention kernels use, measured on the machine that
// runs them, so that a kernel's achieved rate can be read against both the
// published peak and what the chip sustains under the same operand data.
//
//   mfma   v_mfma_f32_32x32x16_bf16 (or, mfma16, v_mfma_f32_16x16x32_bf16)
//          from registers, four (eight) independent
//          accumulator chains, eight distinct operand pairs per wave taken from
//          the caller's buffer (N(0,1) data switches the operand bits the way
//          attention inputs do; constant data does not)
//   exp2   v_exp_f32, sixteen independent chains per lane (x <- 2^-x)
//   fma    v_fma_f32, sixteen independent chains per lane
//   mix    eight exponential chains and 32 FMA chains per lane, one v_exp_f32
//          issued between every four FMAs: if the exponential ran in a unit of
//          its own beside the FMAs, the time would be the larger of the two
//          parts, not their sum
//   lds    ds_read_b128, or the transposing ds_read_b64_tr_b16, from a 64 KiB
//          LDS buffer, conflict-free addresses
//   copy   HBM to HBM, 16-byte loads and stores, four in flight per thread
//
// Every kernel writes one value per thread that depends on all of its work,
// so none of it can be removed by the compiler.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/attn_ceiling.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kOpPairs = 8;     // operand pairs per wave (A and B each)
constexpr int kChains = 16;     // independent VALU chains per lane
constexpr int kLdsChunks = 4096;   // 16-byte LDS chunks (64 KiB)

template <int W>
__global__ __launch_bounds__(W * 64) void mfma_kernel(const bf16x8* __restrict__ ops,
                                                      int64_t op_lanes, float* __restrict__ out,
                                                      int iters) {
  const int64_t gl = (int64_t)blockIdx.x * (W * 64) + threadIdx.x;
  const bf16x8* src = ops + (gl % op_lanes) * (2 * kOpPairs);
  bf16x8 a[kOpPairs], b[kOpPairs];
#pragma unroll
  for (int j = 0; j < kOpPairs; ++j) {
    a[j] = src[j];
    b[j] = src[kOpPairs + j];
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kOpPairs; ++j)
      acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], acc[j & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[gl] = s;
}

// The same stream on v_mfma_f32_16x16x32_bf16: 16 per iteration (the same
// FLOPs as 8 of the 32 x 32 x 16 shape) into 8 independent accumulators.
template <int W>
__global__ __launch_bounds__(W * 64) void mfma16_kernel(const bf16x8* __restrict__ ops,
                                                        int64_t op_lanes, float* __restrict__ out,
                                                        int iters) {
  const int64_t gl = (int64_t)blockIdx.x * (W * 64) + threadIdx.x;
  const bf16x8* src = ops + (gl % op_lanes) * (2 * kOpPairs);
  bf16x8 a[kOpPairs], b[kOpPairs];
#pragma unroll
  for (int j = 0; j < kOpPairs; ++j) {
    a[j] = src[j];
    b[j] = src[kOpPairs + j];
  }
  f32x4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[c][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int j = 0; j < kOpPairs; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b[(j + r) % kOpPairs], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) s += acc[c][i];
  out[gl] = s;
}

__global__ __launch_bounds__(256) void exp2_kernel(float* __restrict__ out, int iters) {
  float x[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) x[j] = 0.5f + 0.01f * j + 1e-5f * threadIdx.x;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);   // stays in [0.5, 1)
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += x[j];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void fma_kernel(float* __restrict__ out, int iters) {
  float x[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) x[j] = 0.5f + 0.01f * j + 1e-5f * threadIdx.x;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) x[j] = __builtin_fmaf(x[j], 0.999f, 0.0005f);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += x[j];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

constexpr int kMixExp = 8, kMixFma = 32;   // chains per lane of the mixed probe

__global__ __launch_bounds__(256) void exp2_fma_kernel(float* __restrict__ out, int iters) {
  float e[kMixExp], f[kMixFma];
#pragma unroll
  for (int j = 0; j < kMixExp; ++j) e[j] = 0.5f + 0.01f * j + 1e-5f * threadIdx.x;
#pragma unroll
  for (int j = 0; j < kMixFma; ++j) f[j] = 0.5f + 0.01f * j + 1e-5f * threadIdx.x;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kMixExp; ++j) {
      e[j] = __builtin_amdgcn_exp2f(-e[j]);
#pragma unroll
      for (int i = 0; i < kMixFma / kMixExp; ++i) {
        const int k = j * (kMixFma / kMixExp) + i;
        f[k] = __builtin_fmaf(f[k], 0.999f, 0.0005f);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kMixExp; ++j) s += e[j];
#pragma unroll
  for (int j = 0; j < kMixFma; ++j) s += f[j];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// 512 threads; each iteration a thread issues 8 reads at its own base plus
// immediate offsets (no address arithmetic in the loop; an empty asm statement
// with a memory clobber keeps the loads inside it, and one that takes each
// result as an operand makes the data arrive without ALU work on it). Plain reads: lane addresses
// are consecutive 16-byte chunks (a wave reads 1 KiB contiguously). Transposing
// reads: consecutive 8-byte pieces (512 bytes per wave).
template <bool TR>
__global__ __launch_bounds__(512) void lds_kernel(float* __restrict__ out, int iters) {
  __shared__ u32x4 buf[kLdsChunks];
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kLdsChunks / 512; ++i) {
    const uint32_t v = (uint32_t)(tid + 512 * i) * 2654435761u;
    buf[tid + 512 * i] = u32x4{v, v ^ 1u, v ^ 2u, v ^ 3u};
  }
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  if constexpr (!TR) {
    const u32x4* base = buf + tid;                 // + 512 i: at most chunk 4095
    u32x4 x[8];
    for (int it = 0; it < iters; ++it) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = base[512 * i];
      // the data must arrive; no ALU work is spent on it
      asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]),
                   "v"(x[6]), "v"(x[7]));
    }
    acc = base[0];
  } else {
    const LDS_AS char* base = (const LDS_AS char*)buf + tid * 8;   // + 4096 i: below 32 KiB
    u32x2 y[8];
    for (int it = 0; it < iters; ++it) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < 8; ++i)
        y[i] = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(base + 4096 * i)));
      asm volatile("" ::"v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3]), "v"(y[4]), "v"(y[5]),
                   "v"(y[6]), "v"(y[7]));
    }
    const u32x2 x = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)base));
    acc.x = x.x;
    acc.y = x.y;
  }
  out[(int64_t)blockIdx.x * 512 + tid] = (float)((acc.x ^ acc.y ^ acc.z ^ acc.w) & 0xFFFF);
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 x0 = src[i], x1 = src[i + stride], x2 = src[i + 2 * stride],
                x3 = src[i + 3 * stride];
    dst[i] = x0;
    dst[i + stride] = x1;
    dst[i + 2 * stride] = x2;
    dst[i + 3 * stride] = x3;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : -3; }

}  // namespace

extern "C" {

int attn_ceiling_mfma_bf16(const void* operands, int64_t operand_lanes, float* out,
                           int workgroups, int waves, int iters, void* stream) {
  if (operands == nullptr || out == nullptr || operand_lanes < 1 || workgroups < 1 ||
      iters < 1 || (waves != 4 && waves != 8) || ((uintptr_t)operands & 15u) != 0)
    return -1;
  (void)hipGetLastError();
  if (waves == 4)
    hipLaunchKernelGGL(mfma_kernel<4>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                       (const bf16x8*)operands, operand_lanes, out, iters);
  else
    hipLaunchKernelGGL(mfma_kernel<8>, dim3(workgroups), dim3(512), 0, (hipStream_t)stream,
                       (const bf16x8*)operands, operand_lanes, out, iters);
  return launched();
}

int attn_ceiling_mfma16_bf16(const void* operands, int64_t operand_lanes, float* out,
                           int workgroups, int waves, int iters, void* stream) {
  if (operands == nullptr || out == nullptr || operand_lanes < 1 || workgroups < 1 ||
      iters < 1 || (waves != 4 && waves != 8) || ((uintptr_t)operands & 15u) != 0)
    return -1;
  (void)hipGetLastError();
  if (waves == 4)
    hipLaunchKernelGGL(mfma16_kernel<4>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                       (const bf16x8*)operands, operand_lanes, out, iters);
  else
    hipLaunchKernelGGL(mfma16_kernel<8>, dim3(workgroups), dim3(512), 0, (hipStream_t)stream,
                       (const bf16x8*)operands, operand_lanes, out, iters);
  return launched();
}

int attn_ceiling_exp2(float* out, int workgroups, int iters, void* stream) {
  if (out == nullptr || workgroups < 1 || iters < 1) return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(exp2_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, out, iters);
  return launched();
}

int attn_ceiling_fma(float* out, int workgroups, int iters, void* stream) {
  if (out == nullptr || workgroups < 1 || iters < 1) return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(fma_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, out, iters);
  return launched();
}

int attn_ceiling_exp2_fma(float* out, int workgroups, int iters, void* stream) {
  if (out == nullptr || workgroups < 1 || iters < 1) return -1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(exp2_fma_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, out,
                     iters);
  return launched();
}

int attn_ceiling_lds_read(float* out, int workgroups, int iters, int transposed, void* stream) {
  if (out == nullptr || workgroups < 1 || iters < 1) return -1;
  (void)hipGetLastError();
  if (transposed)
    hipLaunchKernelGGL(lds_kernel<true>, dim3(workgroups), dim3(512), 0, (hipStream_t)stream, out,
                       iters);
  else
    hipLaunchKernelGGL(lds_kernel<false>, dim3(workgroups), dim3(512), 0, (hipStream_t)stream, out,
                       iters);
  return launched();
}

int attn_ceiling_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  if (dst == nullptr || src == nullptr || bytes < 0 || (bytes & 15) != 0 ||
      ((uintptr_t)dst & 15u) != 0 || ((uintptr_t)src & 15u) != 0)
    return -1;
  if (bytes == 0) return 0;
  (void)hipGetLastError();
  hipLaunchKernelGGL(copy_kernel, dim3(256 * 16), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, (u32x4*)dst, bytes / 16);
  return launched();
}

}  // extern "C"
