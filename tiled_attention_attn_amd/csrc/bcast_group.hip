// Candidate grouping for the in-kernel broadcast attention: a permutation of
// the candidates that puts those of one user next to each other, so that the
// candidates the attention kernel packs into one workgroup usually share a
// user, and with it every K/V read.
//
// Method: "How We Built TLX" (Chinese translation, "Case study 2: in-kernel
// broadcast optimisation for RecSys") reads each user's K/V once for all of
// its candidates. The attention kernel packs short candidates several to a
// workgroup; when they belong to different users, the workgroup runs one pass
// per user with the other candidates' waves idle. Grouping the candidates by
// user first restores one pass per workgroup for any cand2user map.
//
// A counting sort by user in one workgroup: zero the B_u + 1 counters (the
// last one collects users out of range), count, turn the counts into
// starting offsets, then place every candidate at its user's next free
// position. Positions are taken with atomic increments, so the order within
// one user's run is not fixed; any order is valid for the attention kernel,
// whose result does not depend on how candidates are packed. All counter
// traffic goes through device-scope atomics, so every phase reads what the
// previous one wrote after the workgroup barrier between them.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

namespace {

constexpr int kThreads = 1024;

__global__ __launch_bounds__(kThreads) void bcast_group_kernel(const int32_t* __restrict__ c2u,
                                                               int B_c, int B_u,
                                                               int32_t* __restrict__ order,
                                                               int32_t* cnt) {
  const int tid = threadIdx.x;
  const int nb = B_u + 1;   // buckets: one per user, then out of range
  auto bucket = [&](int c) { const int u = c2u[c]; return (u >= 0 && u < B_u) ? u : B_u; };
  for (int i = tid; i < nb; i += kThreads) atomicExch(&cnt[i], 0);
  __syncthreads();
  for (int c = tid; c < B_c; c += kThreads) atomicAdd(&cnt[bucket(c)], 1);
  __syncthreads();
  // Exclusive scan of the counts, kThreads buckets at a time.
  __shared__ int part[kThreads];
  __shared__ int carry;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < nb; base += kThreads) {
    const int i = base + tid;
    const int v = i < nb ? atomicAdd(&cnt[i], 0) : 0;
    part[tid] = v;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int t = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += t;
      __syncthreads();
    }
    if (i < nb) atomicExch(&cnt[i], carry + part[tid] - v);
    __syncthreads();
    if (tid == 0) carry += part[kThreads - 1];
    __syncthreads();
  }
  for (int c = tid; c < B_c; c += kThreads) order[atomicAdd(&cnt[bucket(c)], 1)] = c;
}

}  // namespace

hipError_t launch_bcast_group(const int32_t* cand2user, int B_c, int B_u, int32_t* order,
                              int32_t* work, hipStream_t stream) {
  // An error left pending by an earlier HIP call on this thread is dropped
  // here, so that the status returned after the launch is this launch's.
  (void)hipGetLastError();
  hipLaunchKernelGGL(bcast_group_kernel, dim3(1), dim3(kThreads), 0, stream, cand2user, B_c, B_u,
                     order, work);
  return hipGetLastError();
}

}  // namespace attn
