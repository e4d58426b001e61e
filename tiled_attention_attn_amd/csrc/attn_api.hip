// C ABI front end (include/attn.h): argument checks, work decomposition and
// launch. Every check runs before the first HIP call, so bad arguments are
// reported without touching a device.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/attn.h"
#include "attn_params.h"
#include "gemm_params.h"

namespace attn {
hipError_t launch_ikbo_gemm(GemmParams p, bool gather, bool out_f32, hipStream_t stream);
hipError_t launch_rmsnorm_rows(const void* x, void* y, const float* gamma, float eps, int64_t rows,
                               int D, hipStream_t stream);
hipError_t launch_bf16(const Params& p, int D, bool causal, hipStream_t stream);
hipError_t launch_f32(const Params& p, int D, bool causal, hipStream_t stream);
hipError_t launch_bcast_group(const int32_t* cand2user, int B_c, int B_u, int32_t* order,
                              int32_t* work, hipStream_t stream);
bool plan_bf16(Params& p, int D, bool causal);
}  // namespace attn

// Workspace of the allocation-free entry point: the normalised keys of one
// call, in a file-scope device array each GPU holds from module load until
// the process ends. Host code never uses this name as an address: the
// address is looked up per device (scratch_ptr) and passed to the kernels.
constexpr int64_t kScratchBytes = (int64_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kF32Rows = 64;
constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device: looked up once per device
// (with that device current) and kept. nullptr if the lookup fails.
void* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Shared by both entry points. kv_batches = number of K/V batch entries.
int check_and_launch(const void* q, const void* k, const void* v, void* o,
                     const int32_t* cand2user, int NB, int NKV, int H, int Hkv, int Lq, int Lk,
                     int d, int causal, const int32_t* kv_len, float scale, int dtype,
                     void* stream, const int32_t* q_offsets = nullptr,
                     const int32_t* kv_offsets = nullptr, const uint8_t* block_mask = nullptr,
                     int blk = 0, int mask_heads = 0, const float* gamma_q = nullptr,
                     int qnorm = 0, float eps = 0.f, bool check_only = false,
                     const int32_t* cand_order = nullptr) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_EUNSUPPORTED;
  if (NB < 0 || NKV < 0 || H < 0 || Lq < 0 || Lk < 0 || Hkv < 1) return ATTN_EINVAL;
  if (H % Hkv != 0) return ATTN_EINVAL;
  if (!isfinite(scale) || scale < 0.f) return ATTN_EINVAL;
  if ((int64_t)NB * H * Lq == 0) return ATTN_OK;  // nothing to compute
  if (q == nullptr || o == nullptr) return ATTN_EINVAL;
  if (Lk > 0 && (k == nullptr || v == nullptr || NKV < 1)) return ATTN_EINVAL;
  if (!aligned16(q) || !aligned16(o) || !aligned16(k) || !aligned16(v)) return ATTN_EINVAL;
  // Element counts must stay addressable; grid size must fit an int.
  const int64_t q_elems = (int64_t)NB * H * Lq * d;
  const int64_t kv_elems = (int64_t)NKV * Hkv * Lk * d;
  if (q_elems > ((int64_t)1 << 46) || kv_elems > ((int64_t)1 << 46)) return ATTN_EINVAL;

  attn::Params p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.kv_len = kv_len;
  p.cand2user = cand2user;
  p.cand_order = cand_order;
  p.q_offsets = q_offsets;
  p.kv_offsets = kv_offsets;
  p.block_mask = block_mask;
  if (block_mask != nullptr) {
    p.blk = blk;
    p.nQB = (Lq + blk - 1) / blk;
    p.nKB = (Lk + blk - 1) / blk;
    p.mask_heads = mask_heads;
  }
  p.qnorm = qnorm;
  p.eps = eps;
  p.gamma_q = gamma_q;
  p.NB = NB;
  p.NKV = NKV;
  p.H = H;
  p.Hkv = Hkv;
  p.Lq = Lq;
  p.Lk = Lk;
  const float sc = (scale == 0.f) ? 1.0f / sqrtf((float)d) : scale;
  p.c = sc * 1.4426950408889634f;  // log2(e): the kernels use exp2

  const bool is_causal = causal != 0;
  hipError_t err;
  if (dtype == ATTN_BF16) {
    if (!attn::plan_bf16(p, d, is_causal)) return ATTN_EINVAL;
    if (check_only) return ATTN_OK;
    err = attn::launch_bf16(p, d, is_causal, (hipStream_t)stream);
  } else {
    const int64_t T = (int64_t)NB * H * ((Lq + kF32Rows - 1) / kF32Rows);
    if (T > 0x7fffffff) return ATTN_EINVAL;
    if (check_only) return ATTN_OK;
    p.T = (int)T;
    err = attn::launch_f32(p, d, is_causal, (hipStream_t)stream);
  }
  return err == hipSuccess ? ATTN_OK : ATTN_ELAUNCH;
}

// Attention on RMS-normalised queries and keys (attn_fwd_qknorm). check_only:
// run every argument check and return, launching nothing.
int qknorm(const void* q, const void* k, const void* v, void* o, const float* gamma_q,
           const float* gamma_k, float eps, void* k_norm, int B, int H, int Hkv, int Lq, int Lk,
           int d, int causal, const int32_t* kv_len, float scale, int dtype, void* stream,
           bool check_only) {
  if (dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_EUNSUPPORTED;
  if (!isfinite(eps) || eps < 0.f) return ATTN_EINVAL;
  if (!aligned16(gamma_q) || !aligned16(gamma_k) || !aligned16(k_norm)) return ATTN_EINVAL;
  const bool keys = B > 0 && H > 0 && Lq > 0 && Lk > 0;   // keys to normalise
  if (keys && (k_norm == nullptr || k == nullptr || k_norm == k)) return ATTN_EINVAL;
  // Every other check (shared with attn_fwd) runs before the first launch.
  const int pre = check_and_launch(q, k_norm, v, o, nullptr, B, B, H, Hkv, Lq, Lk, d, causal,
                                   kv_len, scale, dtype, nullptr, nullptr, nullptr, nullptr, 0, 0,
                                   gamma_q, 1, eps, /*check_only=*/true);
  if (pre != ATTN_OK || check_only) return pre;
  if (keys && attn::launch_rmsnorm_rows(k, k_norm, gamma_k, eps, (int64_t)B * Hkv * Lk, d,
                                        (hipStream_t)stream) != hipSuccess)
    return ATTN_ELAUNCH;
  return check_and_launch(q, k_norm, v, o, nullptr, B, B, H, Hkv, Lq, Lk, d, causal, kv_len,
                          scale, dtype, stream, nullptr, nullptr, nullptr, 0, 0, gamma_q, 1, eps);
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int Hkv, int Lq,
             int Lk, int d, int causal, const int32_t* kv_len, float scale, int dtype,
             void* stream) {
  return check_and_launch(q, k, v, o, nullptr, B, B, H, Hkv, Lq, Lk, d, causal, kv_len, scale,
                          dtype, stream);
}

int attn_fwd_bcast(const void* q, const void* k, const void* v, void* o,
                   const int32_t* cand2user, int B_c, int B_u, int H, int Hkv, int Lq, int Lk,
                   int d, int causal, const int32_t* kv_len, float scale, int dtype,
                   void* stream) {
  if (B_c > 0 && B_u < 1) return ATTN_EINVAL;
  if (B_c > 0 && H > 0 && Lq > 0 && cand2user == nullptr) return ATTN_EINVAL;
  return check_and_launch(q, k, v, o, cand2user, B_c, B_u, H, Hkv, Lq, Lk, d, causal, kv_len,
                          scale, dtype, stream);
}

int attn_fwd_bcast_grouped(const void* q, const void* k, const void* v, void* o,
                           const int32_t* cand2user, const int32_t* order, int B_c, int B_u,
                           int H, int Hkv, int Lq, int Lk, int d, int causal,
                           const int32_t* kv_len, float scale, int dtype, void* stream) {
  if (B_c > 0 && B_u < 1) return ATTN_EINVAL;
  if (B_c > 0 && H > 0 && Lq > 0 && (cand2user == nullptr || order == nullptr))
    return ATTN_EINVAL;
  return check_and_launch(q, k, v, o, cand2user, B_c, B_u, H, Hkv, Lq, Lk, d, causal, kv_len,
                          scale, dtype, stream, nullptr, nullptr, nullptr, 0, 0, nullptr, 0,
                          0.f, false, order);
}

int attn_bcast_group(const int32_t* cand2user, int B_c, int B_u, int32_t* order, int32_t* work,
                     void* stream) {
  if (B_c < 0 || B_u < 1 || B_u == 0x7fffffff) return ATTN_EINVAL;
  if (B_c == 0) return ATTN_OK;
  if (cand2user == nullptr || order == nullptr || work == nullptr) return ATTN_EINVAL;
  return attn::launch_bcast_group(cand2user, B_c, B_u, order, work, (hipStream_t)stream) ==
                 hipSuccess
             ? ATTN_OK
             : ATTN_ELAUNCH;
}

int attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o,
                          const uint8_t* block_mask, int mask_heads, int blk, int B, int H,
                          int Hkv, int Lq, int Lk, int d, int causal, const int32_t* kv_len,
                          float scale, int dtype, void* stream) {
  if (blk <= 0 || blk % 128 != 0) return ATTN_EINVAL;
  if (mask_heads != 1 && mask_heads != H) return ATTN_EINVAL;
  if ((int64_t)B * H * Lq == 0) {   // nothing to compute; the other checks still apply
    return check_and_launch(q, k, v, o, nullptr, B, B, H, Hkv, Lq, Lk, d, causal, kv_len, scale,
                            dtype, stream);
  }
  if (block_mask == nullptr) return ATTN_EINVAL;
  if (((int64_t)Lk + blk - 1) / blk > 1024) return ATTN_EINVAL;   // key blocks one list holds
  return check_and_launch(q, k, v, o, nullptr, B, B, H, Hkv, Lq, Lk, d, causal, kv_len, scale,
                          dtype, stream, nullptr, nullptr, block_mask, blk, mask_heads);
}

int attn_fwd_jagged(const void* q, const void* k, const void* v, void* o,
                    const int32_t* q_offsets, const int32_t* kv_offsets, int B, int H, int Hkv,
                    int max_Lq, int max_Lk, int d, int causal, float scale, int dtype,
                    void* stream) {
  if (B > 0 && H > 0 && max_Lq > 0 && (q_offsets == nullptr || kv_offsets == nullptr))
    return ATTN_EINVAL;
  return check_and_launch(q, k, v, o, nullptr, B, B, H, Hkv, max_Lq, max_Lk, d, causal, nullptr,
                          scale, dtype, stream, q_offsets, kv_offsets);
}

int attn_fwd_qknorm(const void* q, const void* k, const void* v, void* o, const float* gamma_q,
                    const float* gamma_k, float eps, void* k_norm, int B, int H, int Hkv, int Lq,
                    int Lk, int d, int causal, const int32_t* kv_len, float scale, int dtype,
                    void* stream) {
  return qknorm(q, k, v, o, gamma_q, gamma_k, eps, k_norm, B, H, Hkv, Lq, Lk, d, causal, kv_len,
                scale, dtype, stream, false);
}

int attn_fwd_qknorm_noalloc(const void* q, const void* k, const void* v, void* o,
                            const float* gamma_q, const float* gamma_k, float eps, int B, int H,
                            int Hkv, int Lq, int Lk, int d, int causal, const int32_t* kv_len,
                            float scale, int dtype, void* stream) {
  const bool keys = B > 0 && H > 0 && Lq > 0 && Lk > 0;
  // Every argument check of attn_fwd_qknorm runs first (an aligned stand-in
  // for the workspace, never dereferenced: check_only launches nothing), then
  // the size limit, and only then the one HIP call that finds the array.
  const int pre = qknorm(q, k, v, o, gamma_q, gamma_k, eps, keys ? (void*)(uintptr_t)256 : nullptr,
                         B, H, Hkv, Lq, Lk, d, causal, kv_len, scale, dtype, stream, true);
  if (pre != ATTN_OK) return pre;
  if (!keys)   // no key to normalise: the attention pass alone (zero rows when Lk == 0)
    return qknorm(q, k, v, o, gamma_q, gamma_k, eps, nullptr, B, H, Hkv, Lq, Lk, d, causal,
                  kv_len, scale, dtype, stream, false);
  if ((int64_t)B * Hkv * Lk * d * 2 > kScratchBytes) return ATTN_ESCRATCH;
  void* ws = scratch_ptr();
  if (ws == nullptr) return ATTN_ELAUNCH;
  return qknorm(q, k, v, o, gamma_q, gamma_k, eps, ws, B, H, Hkv, Lq, Lk, d, causal, kv_len,
                scale, dtype, stream, false);
}

int ikbo_linear(const void* x_user, const void* x_cand, const void* w, const float* bias,
                const int32_t* cand2user, void* y, float* z, int B_u, int B_c, int K_u, int K_c,
                int N, int y_dtype, void* stream) {
  if (y_dtype != ATTN_F32 && y_dtype != ATTN_BF16) return ATTN_EUNSUPPORTED;
  if (B_u < 0 || B_c < 0 || K_u < 0 || K_c < 0 || N < 0) return ATTN_EINVAL;
  if (K_u % 8 != 0 || K_c % 8 != 0 || N % 4 != 0) return ATTN_EINVAL;
  const int64_t K = (int64_t)K_u + K_c;
  if (K > ((int64_t)1 << 20)) return ATTN_EINVAL;
  if (B_c > 0 && N > 0 && B_u < 1) return ATTN_EINVAL;
  if (N == 0 || (B_u == 0 && B_c == 0)) return ATTN_OK;
  // Weight rows are addressed with 32-bit offsets; activations are split by rows.
  if ((int64_t)(N - 1) * K * 2 + K * 2 > 0x7fffffff) return ATTN_EINVAL;
  // bf16 output is stored with 32-bit offsets within 256-row tiles.
  if (y_dtype == ATTN_BF16 && B_c > 0 && N >= (1 << 22)) return ATTN_EINVAL;
  if ((int64_t)B_c * N > ((int64_t)1 << 46) || (int64_t)B_u * N > ((int64_t)1 << 46))
    return ATTN_EINVAL;
  auto need = [](const void* ptr, bool used) { return !used || (ptr != nullptr && aligned16(ptr)); };
  if (!need(z, B_u > 0) || !need(x_user, B_u > 0 && K_u > 0) || !need(w, K > 0) ||
      !need(x_cand, B_c > 0 && K_c > 0) || !need(y, B_c > 0) || !need(cand2user, B_c > 0) ||
      !aligned16(bias))
    return ATTN_EINVAL;

  attn::GemmParams p{};
  p.N = N;
  p.ldb = (int)K;
  hipError_t err = hipSuccess;
  if (B_u > 0) {   // z = x_user w_user^T + bias
    p.a = x_user;
    p.b = w;
    p.c = z;
    p.bias = bias;
    p.M = B_u;
    p.K = K_u;
    p.lda = K_u;
    err = attn::launch_ikbo_gemm(p, false, true, (hipStream_t)stream);
  }
  if (err == hipSuccess && B_c > 0) {   // y = x_cand w_cand^T + z[cand2user]
    p.a = x_cand;
    p.b = (const char*)w + (size_t)K_u * 2;
    p.c = y;
    p.bias = nullptr;
    p.z = z;
    p.zrow = cand2user;
    p.Mz = B_u;
    p.M = B_c;
    p.K = K_c;
    p.lda = K_c;
    err = attn::launch_ikbo_gemm(p, true, y_dtype == ATTN_F32, (hipStream_t)stream);
  }
  return err == hipSuccess ? ATTN_OK : ATTN_ELAUNCH;
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_EUNSUPPORTED: return "unsupported head dimension or dtype";
    case ATTN_ELAUNCH: return "kernel launch failed";
    case ATTN_ESCRATCH:
      return "problem needs more than the allocation-free entry point's 32 MiB workspace";
    default: return "unknown status";
  }
}

int attn_version(void) { return 106; }

}  // extern "C"
