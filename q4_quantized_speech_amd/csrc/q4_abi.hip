// C ABI of the Q4_0 library (declared in include/q4.h): argument validation,
// then one launch on the caller's stream.  No allocation, no synchronisation.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/q4.h"
#include "q4_kernels.h"

namespace q4 {

namespace {
thread_local int g_last_hip_error = 0;
constexpr int kMaxDevices = 64;
// 0 = not cached yet.  Threads that race on the first call all store the
// same value; atomics keep that free of data races.
std::atomic<int> g_cu_count[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

q4_status hip_status(hipError_t e) {
  if (e == hipSuccess) return Q4_OK;
  g_last_hip_error = static_cast<int>(e);
  return Q4_ERR_HIP;
}

bool k_ok(int64_t K) { return K > 0 && K % 32 == 0 && K <= (int64_t(1) << 30); }

bool matmul_shape_ok(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= int64_t(65535) * 128 && N >= 1 && N < (int64_t(1) << 31) && k_ok(K) &&
         K <= (int64_t(1) << 22) && N * K < (int64_t(1) << 40) && M * K < (int64_t(1) << 40) &&
         M * N < (int64_t(1) << 40);
}
}  // namespace

DeviceInfo device_info() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DeviceInfo{256};
  int cu = g_cu_count[dev].load(std::memory_order_relaxed);
  if (cu == 0) {
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
      cu = 256;
    g_cu_count[dev].store(cu, std::memory_order_relaxed);
  }
  return DeviceInfo{cu};
}

}  // namespace q4

using namespace q4;

extern "C" {

int q4_abi_version(void) { return 3; }

const char* q4_status_string(q4_status status) {
  switch (status) {
    case Q4_OK: return "ok";
    case Q4_ERR_NULL: return "a required pointer is NULL";
    case Q4_ERR_SHAPE: return "M, N or K out of range (K must be a positive multiple of 32)";
    case Q4_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case Q4_ERR_WORKSPACE: return "workspace missing or too small";
    case Q4_ERR_HIP: return "a HIP call failed (see q4_last_hip_error)";
    case Q4_ERR_FORMAT: return "malformed or unsupported GGUF content";
    case Q4_ERR_IO: return "a file could not be opened or read";
    case Q4_ERR_NOT_FOUND: return "no such tensor, metadata key or index";
    default: return "unknown status";
  }
}

int q4_last_hip_error(void) { return g_last_hip_error; }

size_t q4_row_bytes(int64_t K) {
  if (!k_ok(K)) return 0;
  return static_cast<size_t>(K / 32) * 18;
}

q4_status q4_matvec(const void* w_q4, const float* x, float* y, int64_t M, int64_t N, int64_t K,
                    void* stream) {
  if (!w_q4 || !x || !y) return Q4_ERR_NULL;
  if (M < 1 || M > 8 || N < 1 || N >= (int64_t(1) << 31) || !k_ok(K) || N * K >= (int64_t(1) << 40))
    return Q4_ERR_SHAPE;
  if (!aligned16(w_q4) || !aligned16(x) || !aligned16(y)) return Q4_ERR_ALIGN;
  return hip_status(launch_matvec(static_cast<const uint8_t*>(w_q4), x, y, M, N, K,
                                  static_cast<hipStream_t>(stream)));
}

size_t q4_matmul_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!matmul_shape_ok(M, N, K)) return 0;
  return matmul_workspace_bytes(M, N, K, device_info().cu_count);
}

q4_status q4_matmul(const void* w_q4, const float* x, float* y, int64_t M, int64_t N, int64_t K,
                    void* workspace, size_t ws_bytes, void* stream) {
  if (!w_q4 || !x || !y) return Q4_ERR_NULL;
  if (!matmul_shape_ok(M, N, K)) return Q4_ERR_SHAPE;
  if (!aligned16(w_q4) || !aligned16(x) || !aligned16(y) || (workspace && !aligned16(workspace)))
    return Q4_ERR_ALIGN;
  return hip_status(launch_matmul(static_cast<const uint8_t*>(w_q4), x, y, nullptr, M, N, K,
                                  workspace, workspace ? ws_bytes : 0, device_info().cu_count,
                                  static_cast<hipStream_t>(stream)));
}

size_t q4_matmul_residual_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!matmul_shape_ok(M, N, K)) return 0;
  return matmul_residual_workspace_bytes(M, N, K, device_info().cu_count);
}

q4_status q4_matmul_residual(const void* w_q4, const float* x, const float* r, float* y,
                             int64_t M, int64_t N, int64_t K, void* workspace, size_t ws_bytes,
                             void* stream) {
  if (!w_q4 || !x || !r || !y) return Q4_ERR_NULL;
  if (!matmul_shape_ok(M, N, K)) return Q4_ERR_SHAPE;
  if (!aligned16(w_q4) || !aligned16(x) || !aligned16(r) || !aligned16(y) ||
      (workspace && !aligned16(workspace)))
    return Q4_ERR_ALIGN;
  const size_t wsb = workspace ? ws_bytes : 0;
  const int cus = device_info().cu_count;
  if (r == y && !matmul_residual_fused(M, N, K, wsb, cus) &&
      wsb < static_cast<size_t>(M) * static_cast<size_t>(N) * sizeof(float))
    return Q4_ERR_WORKSPACE;
  return hip_status(launch_matmul(static_cast<const uint8_t*>(w_q4), x, y, r, M, N, K, workspace,
                                  wsb, cus, static_cast<hipStream_t>(stream)));
}

q4_status q4_embed_rows(const void* table_q4, const int32_t* ids, float* out, int64_t M, int64_t N,
                        int64_t K, void* stream) {
  if (!table_q4 || !ids || !out) return Q4_ERR_NULL;
  if (M < 1 || M >= (int64_t(1) << 31) || N < 1 || N >= (int64_t(1) << 31) || !k_ok(K) ||
      M * (K / 32) >= (int64_t(1) << 40) || N * K >= (int64_t(1) << 40))
    return Q4_ERR_SHAPE;
  if (!aligned16(table_q4) || !aligned16(ids) || !aligned16(out)) return Q4_ERR_ALIGN;
  return hip_status(launch_embed(static_cast<const uint8_t*>(table_q4), ids, out, M, N, K,
                                 static_cast<hipStream_t>(stream)));
}

size_t q4_lmhead_argmax_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  (void)N;
  (void)K;
  if (M < 1 || M > 64) return 0;
  return lmhead_workspace_bytes(M);
}

q4_status q4_lmhead_argmax(const void* w_q4, const float* x, int32_t* out_idx, float* out_val,
                           int64_t M, int64_t N, int64_t K, void* workspace, size_t ws_bytes,
                           void* stream) {
  if (!w_q4 || !x || !out_idx) return Q4_ERR_NULL;
  if (M < 1 || M > 64 || N < 1 || N >= (int64_t(1) << 31) || !k_ok(K) || N * K >= (int64_t(1) << 40))
    return Q4_ERR_SHAPE;
  if (!aligned16(w_q4) || !aligned16(x) || !aligned16(out_idx) || (out_val && !aligned16(out_val)))
    return Q4_ERR_ALIGN;
  if (!workspace || ws_bytes < lmhead_workspace_bytes(M)) return Q4_ERR_WORKSPACE;
  if (!aligned16(workspace)) return Q4_ERR_ALIGN;
  return hip_status(launch_lmhead_argmax(static_cast<const uint8_t*>(w_q4), x, out_idx, out_val,
                                         nullptr, M, N, K, workspace,
                                         static_cast<hipStream_t>(stream)));
}

const char* q4_matmul_route(int64_t M, int64_t N, int64_t K, size_t ws_bytes, int32_t* splits) {
  if (!matmul_shape_ok(M, N, K)) return nullptr;
  int sp = 1;
  const char* r = matmul_route(M, N, K, ws_bytes, device_info().cu_count, &sp);
  if (splits) *splits = sp;
  return r;
}

const char* q4_matvec_route(int64_t N, int64_t K, int32_t argmax) {
  if (N < 1 || N >= (int64_t(1) << 31) || !k_ok(K) || N * K >= (int64_t(1) << 40)) return nullptr;
  return matvec_route(N, K, argmax != 0);
}

q4_status q4_decode_chain(const q4_matvec_step* steps, int64_t nsteps, const void* table_q4,
                          int64_t vocab, int64_t dim, const float* head_x, int32_t* out_idx,
                          float* out_val, float* out_embed, void* workspace, size_t ws_bytes,
                          void* stream) {
  if (nsteps < 0 || nsteps > Q4_CHAIN_MAX_STEPS) return Q4_ERR_SHAPE;
  if (nsteps > 0 && !steps) return Q4_ERR_NULL;
  if (nsteps == 0 && !table_q4) return Q4_ERR_SHAPE;  // nothing to do
  for (int64_t i = 0; i < nsteps; ++i) {
    const q4_matvec_step& st = steps[i];
    if (!st.w_q4 || !st.x || !st.y) return Q4_ERR_NULL;
    if (st.N < 1 || st.N >= (int64_t(1) << 31) || !k_ok(st.K) || st.N * st.K >= (int64_t(1) << 40))
      return Q4_ERR_SHAPE;
    if (!aligned16(st.w_q4) || !aligned16(st.x) || !aligned16(st.y)) return Q4_ERR_ALIGN;
  }
  if (table_q4) {
    if (!head_x || !out_idx) return Q4_ERR_NULL;
    if (vocab < 1 || vocab >= (int64_t(1) << 31) || !k_ok(dim) || vocab * dim >= (int64_t(1) << 40))
      return Q4_ERR_SHAPE;
    if (!aligned16(table_q4) || !aligned16(head_x) || !aligned16(out_idx) ||
        (out_val && !aligned16(out_val)) || (out_embed && !aligned16(out_embed)))
      return Q4_ERR_ALIGN;
    if (!workspace || ws_bytes < lmhead_workspace_bytes(1)) return Q4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return Q4_ERR_ALIGN;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t i = 0; i < nsteps; ++i) {
    const q4_matvec_step& st = steps[i];
    const hipError_t e = launch_matvec(static_cast<const uint8_t*>(st.w_q4), st.x, st.y, 1, st.N,
                                       st.K, s);
    if (e != hipSuccess) return hip_status(e);
  }
  if (!table_q4) return Q4_OK;
  return hip_status(launch_lmhead_argmax(static_cast<const uint8_t*>(table_q4), head_x, out_idx,
                                         out_val, out_embed, 1, vocab, dim, workspace, s));
}

q4_status q4_lmhead_argmax_noalloc(const void* w_q4, const float* x, int32_t* out_idx,
                                   float* out_val, int64_t M, int64_t N, int64_t K, void* stream) {
  if (!w_q4 || !x || !out_idx) return Q4_ERR_NULL;
  if (M < 1 || M > lmhead_noalloc_max_m() || N < 1 || N >= (int64_t(1) << 31) || !k_ok(K) ||
      N * K >= (int64_t(1) << 40))
    return Q4_ERR_SHAPE;
  if (!aligned16(w_q4) || !aligned16(x) || !aligned16(out_idx) || (out_val && !aligned16(out_val)))
    return Q4_ERR_ALIGN;
  return hip_status(launch_lmhead_argmax_noalloc(static_cast<const uint8_t*>(w_q4), x, out_idx,
                                                 out_val, M, N, K, static_cast<hipStream_t>(stream)));
}

q4_status q4_quantize(const float* w, void* w_q4, int64_t N, int64_t K, int32_t* flag,
                      void* stream) {
  if (!w || !w_q4) return Q4_ERR_NULL;
  // N is bounded before the product (K / 32 <= 2^25), so nothing overflows
  if (N < 1 || N >= (int64_t(1) << 37) || !k_ok(K) || N * (K / 32) >= (int64_t(1) << 37))
    return Q4_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(w_q4) || (flag && (reinterpret_cast<uintptr_t>(flag) & 3u)))
    return Q4_ERR_ALIGN;
  return hip_status(launch_quantize(w, static_cast<uint8_t*>(w_q4), N, K, flag,
                                    static_cast<hipStream_t>(stream)));
}

}  // extern "C"
