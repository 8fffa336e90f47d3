// Host-side launchers of the gfx950 kernels (internal to the library; the
// public surface is include/q4.h).  Each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

struct DeviceInfo {
  int cu_count;
};
DeviceInfo device_info();

hipError_t launch_matvec(const uint8_t* w, const float* x, float* y, int64_t M, int64_t N,
                         int64_t K, hipStream_t s);

// out_embed (nullable): the decoded table row of each chosen index, [M, K].
hipError_t launch_lmhead_argmax(const uint8_t* w, const float* x, int32_t* out_idx, float* out_val,
                                float* out_embed, int64_t M, int64_t N, int64_t K, void* workspace,
                                hipStream_t s);
size_t lmhead_workspace_bytes(int64_t M);
// The argmax with the library's own per-device scratch (no allocation);
// 1 <= M <= lmhead_noalloc_max_m().
int64_t lmhead_noalloc_max_m();
hipError_t launch_lmhead_argmax_noalloc(const uint8_t* w, const float* x, int32_t* out_idx,
                                        float* out_val, int64_t M, int64_t N, int64_t K,
                                        hipStream_t s);
// Name of the matvec kernel variant launched for (N, K) (argmax or not).
const char* matvec_route(int64_t N, int64_t K, bool argmax);
// Name of the matmul kernel launched for the shape and workspace size, and
// its K split count.
const char* matmul_route(int64_t M, int64_t N, int64_t K, size_t ws_bytes, int cus, int* splits);

// r (nullable): y = r + the product (r is y or does not overlap it); an
// unfused route in place needs M*N floats of workspace for the product.
hipError_t launch_matmul(const uint8_t* w, const float* x, float* y, const float* r, int64_t M,
                         int64_t N, int64_t K, void* ws, size_t ws_bytes, int cus, hipStream_t s);
size_t matmul_workspace_bytes(int64_t M, int64_t N, int64_t K, int cus);
// Whether the residual add rides in a kernel of the product for this plan.
bool matmul_residual_fused(int64_t M, int64_t N, int64_t K, size_t ws_bytes, int cus);
size_t matmul_residual_workspace_bytes(int64_t M, int64_t N, int64_t K, int cus);
// M <= 4, K % 64 == 0: pps (pairs of blocks per K split) a multiple of 4
// when splits > 1; partials [splits][M][N] in P, folded by the caller.
int matmul_small_per_cu();
void launch_matmul_small(const uint8_t* w, const float* x, float* y, float* P, int64_t M,
                         int64_t N, int64_t K, int splits, int pps, hipStream_t s);

// 5 <= M <= 16: chunks of 256 K values per wave of the stream16 kernel
// (0 when it does not serve the shape), and its launch (no workspace).
int matmul_stream16_chunks(int64_t M, int64_t K);
hipError_t launch_matmul_stream16(const uint8_t* w, const float* x, float* y, int64_t M,
                                  int64_t N, int64_t K, int cus, hipStream_t s);

hipError_t launch_embed(const uint8_t* table, const int32_t* ids, float* out, int64_t M,
                        int64_t N, int64_t K, hipStream_t s);

hipError_t launch_quantize(const float* w, uint8_t* out, int64_t N, int64_t K, int32_t* flag,
                           hipStream_t s);

}  // namespace q4
