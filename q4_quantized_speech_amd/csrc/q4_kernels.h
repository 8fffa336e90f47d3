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

hipError_t launch_lmhead_argmax(const uint8_t* w, const float* x, int32_t* out_idx, float* out_val,
                                int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t s);
size_t lmhead_workspace_bytes(int64_t M);

hipError_t launch_matmul(const uint8_t* w, const float* x, float* y, int64_t M, int64_t N,
                         int64_t K, void* ws, size_t ws_bytes, int cus, hipStream_t s);
size_t matmul_workspace_bytes(int64_t M, int64_t N, int64_t K, int cus);
// M <= 4, K % 64 == 0: pps (pairs of blocks per K split) a multiple of 4
// when splits > 1; partials [splits][M][N] in P, folded by the caller.
int matmul_small_per_cu();
void launch_matmul_small(const uint8_t* w, const float* x, float* y, float* P, int64_t M,
                         int64_t N, int64_t K, int splits, int pps, hipStream_t s);

hipError_t launch_embed(const uint8_t* table, const int32_t* ids, float* out, int64_t M,
                        int64_t N, int64_t K, hipStream_t s);

hipError_t launch_quantize(const float* w, uint8_t* out, int64_t N, int64_t K, int32_t* flag,
                           hipStream_t s);

}  // namespace q4
