// Q4_0 matrix-vector product (decode step, M = 1) and the LM-head argmax.
//
// Section "Architecture" of "Implémentation en Rust du modèle Voxtral Mini 4B
// Realtime de Mistral pour l'exécuter dans le navigateur": every decoder
// projection runs on Q4_0 weights; per generated token each weight byte is read
// once, so this kernel is an HBM stream.  Design for gfx950:
//  * the weight matrix is read as 36-byte block pairs (two Q4_0 blocks; a pair
//    whose first block has an even flat index is dword aligned), 16 lanes per
//    row, so each 16-lane DPP row reads 576 contiguous bytes per step;
//  * x is staged once per workgroup in LDS with the per-block sums
//    S_b = sum of x over block b, padded to 272 bytes per pair so that the 16
//    lanes of a row read 16 different pairs without bank conflicts;
//  * codes are turned into floats with v_cvt_f32_ubyte (one op per weight) and
//    accumulated as sum q*x; the -8 offset is applied per block:
//    y += d * (sum_j q_j x_j - 8 * S_b);
//  * the 16 partial sums of a row are reduced inside the DPP row;
//  * workgroups are persistent (a grid-stride loop over row groups) so x is
//    staged once per workgroup however tall the matrix is.
// The argmax variant ("LM head" over the same 131072-row table the embedding
// lookup of section "Solutions techniques", item 3, reads) keeps the best
// (value, lowest index) per lane, reduces it per workgroup, and the last
// workgroup to finish reduces the per-workgroup partials in a fixed order.

#include "q4_device.h"
#include "q4_kernels.h"

namespace q4 {
namespace {

constexpr int MV_THREADS = 256;
constexpr int XP = 68;                 // floats per staged pair: 64 x + S_0, S_1, pad
constexpr int MAX_LDS_K = 15360;       // K with (K/64)*272 B <= 64 KiB
constexpr int AM_MAX_PARTIALS = 2048;  // per-row partials of the argmax reduction

typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));

// Stage x[0..K) and the block sums into LDS (layout: pair c at xs + 68c).
__device__ __forceinline__ void stage_x(const float* __restrict__ x, float* xs, int nb) {
  for (int b = threadIdx.x; b < nb; b += blockDim.x) {
    const f32x4* src = reinterpret_cast<const f32x4*>(x + static_cast<int64_t>(b) * QK);
    float* dst = xs + (b >> 1) * XP + (b & 1) * QK;
    f32x4 v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = src[t];
    f32x4 s4 = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
#pragma unroll
    for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(dst + 4 * t) = v[t];
    xs[(b >> 1) * XP + 64 + (b & 1)] = (s4.x + s4.y) + (s4.z + s4.w);
  }
}

// One block pair of one row against the staged x: returns
// d0*(sum q x - 8 S0) + d1*(sum q x - 8 S1) for R rows at once.
template <int R>
__device__ __forceinline__ void pair_dot(const uint32_t (&w)[R][9], const float* xp, float (&acc)[R]) {
  float s0[R], s1[R];
#pragma unroll
  for (int r = 0; r < R; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const f32x4 xl = *reinterpret_cast<const f32x4*>(xp + 4 * t);
    const f32x4 xh = *reinterpret_cast<const f32x4*>(xp + 16 + 4 * t);
#pragma unroll
    for (int r = 0; r < R; ++r) s0[r] = nib_dot4(shift16(w[r][t + 1], w[r][t]), xl, xh, s0[r]);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const f32x4 xl = *reinterpret_cast<const f32x4*>(xp + 32 + 4 * t);
    const f32x4 xh = *reinterpret_cast<const f32x4*>(xp + 48 + 4 * t);
#pragma unroll
    for (int r = 0; r < R; ++r) s1[r] = nib_dot4(w[r][5 + t], xl, xh, s1[r]);
  }
  const float S0 = xp[64], S1 = xp[65];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float d0 = half_bits_to_float(w[r][0] & 0xFFFFu);
    const float d1 = half_bits_to_float(w[r][4] >> 16);
    acc[r] = __builtin_fmaf(d0, __builtin_fmaf(-8.f, S0, s0[r]), acc[r]);
    acc[r] = __builtin_fmaf(d1, __builtin_fmaf(-8.f, S1, s1[r]), acc[r]);
  }
}

template <int R>
__device__ __forceinline__ void load_pairs(const uint8_t* __restrict__ W, const int64_t (&row)[R],
                                           const bool (&ok)[R], int64_t row_bytes, int c,
                                           uint32_t (&w)[R][9]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (ok[r]) {
      const uint8_t* p = W + row[r] * row_bytes + static_cast<int64_t>(c) * PAIR_BYTES;
      const u32x4a a = *reinterpret_cast<const u32x4a*>(p);
      const u32x4a b = *reinterpret_cast<const u32x4a*>(p + 16);
      w[r][0] = a.x; w[r][1] = a.y; w[r][2] = a.z; w[r][3] = a.w;
      w[r][4] = b.x; w[r][5] = b.y; w[r][6] = b.z; w[r][7] = b.w;
      w[r][8] = *reinterpret_cast<const uint32_t*>(p + 32);
    } else {
#pragma unroll
      for (int t = 0; t < 9; ++t) w[r][t] = 0u;
    }
  }
}

// Argmax bookkeeping: idx < 0 means "no candidate"; NaN never wins.
__device__ __forceinline__ bool am_better(float v, int i, float bv, int bi) {
  if (bi < 0) return !(v != v);
  return v > bv || (v == bv && i < bi);
}

// Fold the candidates of all threads of the workgroup; result valid in thread 0.
__device__ __forceinline__ void am_block_reduce(float& bv, int& bi) {
  __shared__ float sv[MV_THREADS / 16];
  __shared__ int si[MV_THREADS / 16];
  // within a 16-lane row
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 16);
    const int oi = __shfl_xor(bi, o, 16);
    if (am_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  const int grp = threadIdx.x >> 4;
  if ((threadIdx.x & 15) == 0) { sv[grp] = bv; si[grp] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int g = 1; g < static_cast<int>(blockDim.x >> 4); ++g)
      if (am_better(sv[g], si[g], bv, bi)) { bv = sv[g]; bi = si[g]; }
  }
}

// Workspace layout: counters [64] uint32 (256 B), then partials
// [M][AM_MAX_PARTIALS] of uint64 {low: float bits of the value, high: index}.
__device__ __forceinline__ void am_finish(float bv, int bi, int m, int32_t* out_idx, float* out_val,
                                          void* workspace) {
  unsigned* counters = reinterpret_cast<unsigned*>(workspace);
  uint64_t* partials = reinterpret_cast<uint64_t*>(reinterpret_cast<uint8_t*>(workspace) + 256) +
                       static_cast<int64_t>(m) * AM_MAX_PARTIALS;
  __shared__ int s_last;
  am_block_reduce(bv, bi);
  if (threadIdx.x == 0) {
    partials[blockIdx.x] = static_cast<uint64_t>(__float_as_uint(bv)) |
                           (static_cast<uint64_t>(static_cast<uint32_t>(bi)) << 32);
    __threadfence();
    const unsigned t = atomicAdd(&counters[m], 1u);
    s_last = (t == gridDim.x - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  float v = 0.f;
  int i = -1;
  for (int p = threadIdx.x; p < static_cast<int>(gridDim.x); p += blockDim.x) {
    const uint64_t e = __builtin_nontemporal_load(&partials[p]);
    const float ev = __uint_as_float(static_cast<uint32_t>(e));
    const int ei = static_cast<int>(static_cast<uint32_t>(e >> 32));
    if (am_better(ev, ei, v, i)) { v = ev; i = ei; }
  }
  am_block_reduce(v, i);
  if (threadIdx.x == 0) {
    out_idx[m] = i;
    if (out_val) out_val[m] = i >= 0 ? v : __builtin_nanf("");
    counters[m] = 0u;  // leave the workspace zero for the next call
  }
}

// Pair kernel: K % 64 == 0 and K <= MAX_LDS_K.  Each wave holds 4 groups of
// 16 lanes; group g handles R rows; a pass of the workgroup covers 16R rows.
template <int R, bool ARGMAX>
__global__ __launch_bounds__(MV_THREADS) void matvec_pairs_kernel(
    const uint8_t* __restrict__ W, const float* __restrict__ X, float* __restrict__ Y,
    int32_t* __restrict__ out_idx, float* __restrict__ out_val, void* workspace, int64_t N,
    int K) {
  extern __shared__ float xs[];
  const int m = blockIdx.y;
  const int nb = K / QK, nbp = nb / 2;
  const int64_t row_bytes = static_cast<int64_t>(nbp) * PAIR_BYTES;
  stage_x(X + static_cast<int64_t>(m) * K, xs, nb);
  __syncthreads();

  const int j = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;  // 0..15 over the workgroup
  const int64_t rows_per_pass = 16 * R;
  float bv = 0.f;
  int bi = -1;
  for (int64_t row0 = static_cast<int64_t>(blockIdx.x) * rows_per_pass; row0 < N;
       row0 += static_cast<int64_t>(gridDim.x) * rows_per_pass) {
    int64_t row[R];
    bool ok[R];
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      row[r] = row0 + grp * R + r;
      ok[r] = row[r] < N;
      acc[r] = 0.f;
    }
    uint32_t w[R][9];
    if (j < nbp) load_pairs<R>(W, row, ok, row_bytes, j, w);
    for (int c = j; c < nbp; c += 16) {
      uint32_t wn[R][9];
      const bool more = c + 16 < nbp;
      if (more) load_pairs<R>(W, row, ok, row_bytes, c + 16, wn);
      pair_dot<R>(w, xs + c * XP, acc);
      if (more) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int t = 0; t < 9; ++t) w[r][t] = wn[r][t];
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float v = row16_sum(acc[r]);
      if constexpr (ARGMAX) {
        if (ok[r] && am_better(v, static_cast<int>(row[r]), bv, bi)) { bv = v; bi = static_cast<int>(row[r]); }
      } else {
        if (ok[r] && j == 0) Y[static_cast<int64_t>(m) * N + row[r]] = v;
      }
    }
  }
  if constexpr (ARGMAX) am_finish(bv, bi, m, out_idx, out_val, workspace);
}

// Generic kernel: any K % 32 == 0 (odd block counts, very long rows).  16
// lanes per row, one block per lane per step, x read from global memory.
template <bool ARGMAX>
__global__ __launch_bounds__(MV_THREADS) void matvec_any_kernel(
    const uint8_t* __restrict__ W, const float* __restrict__ X, float* __restrict__ Y,
    int32_t* __restrict__ out_idx, float* __restrict__ out_val, void* workspace, int64_t N,
    int K) {
  const int m = blockIdx.y;
  const float* x = X + static_cast<int64_t>(m) * K;
  const int nb = K / QK;
  const int j = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;
  float bv = 0.f;
  int bi = -1;
  for (int64_t row0 = static_cast<int64_t>(blockIdx.x) * 16; row0 < N;
       row0 += static_cast<int64_t>(gridDim.x) * 16) {
    const int64_t row = row0 + grp;
    const bool ok = row < N;
    float acc = 0.f;
    if (ok) {
      for (int b = j; b < nb; b += 16) {
        uint32_t d16, qs[4];
        load_block_any(W, row * nb + b, d16, qs);
        const f32x4* xb = reinterpret_cast<const f32x4*>(x + static_cast<int64_t>(b) * QK);
        float s = 0.f, S = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x4 xl = xb[t], xh = xb[4 + t];
          s = nib_dot4(qs[t], xl, xh, s);
          S += (xl.x + xl.y) + (xl.z + xl.w) + ((xh.x + xh.y) + (xh.z + xh.w));
        }
        acc = __builtin_fmaf(half_bits_to_float(d16), __builtin_fmaf(-8.f, S, s), acc);
      }
    }
    const float v = row16_sum(acc);
    if constexpr (ARGMAX) {
      if (ok && am_better(v, static_cast<int>(row), bv, bi)) { bv = v; bi = static_cast<int>(row); }
    } else {
      if (ok && j == 0) Y[static_cast<int64_t>(m) * N + row] = v;
    }
  }
  if constexpr (ARGMAX) am_finish(bv, bi, m, out_idx, out_val, workspace);
}

int persistent_blocks(int64_t passes, int per_cu) {
  const int64_t cap = static_cast<int64_t>(device_info().cu_count) * per_cu;
  return static_cast<int>(passes < cap ? passes : cap);
}

template <bool ARGMAX>
hipError_t launch_mv(const uint8_t* w, const float* x, float* y, int32_t* idx, float* val,
                     void* ws, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  const bool pairs = (K % 64 == 0) && K <= MAX_LDS_K;
  if (pairs) {
    const size_t lds = static_cast<size_t>(K / 64) * XP * sizeof(float);
    // two rows per lane once the matrix is tall enough to keep every CU busy
    const bool tall = N >= static_cast<int64_t>(device_info().cu_count) * 64;
    if (tall) {
      int g = persistent_blocks((N + 31) / 32, 4);
      if (ARGMAX && g > AM_MAX_PARTIALS) g = AM_MAX_PARTIALS;
      hipLaunchKernelGGL((matvec_pairs_kernel<2, ARGMAX>), dim3(g, M), dim3(MV_THREADS), lds, s,
                         w, x, y, idx, val, ws, N, static_cast<int>(K));
    } else {
      int g = persistent_blocks((N + 15) / 16, 4);
      if (ARGMAX && g > AM_MAX_PARTIALS) g = AM_MAX_PARTIALS;
      hipLaunchKernelGGL((matvec_pairs_kernel<1, ARGMAX>), dim3(g, M), dim3(MV_THREADS), lds, s,
                         w, x, y, idx, val, ws, N, static_cast<int>(K));
    }
  } else {
    int g = persistent_blocks((N + 15) / 16, 8);
    if (ARGMAX && g > AM_MAX_PARTIALS) g = AM_MAX_PARTIALS;
    hipLaunchKernelGGL((matvec_any_kernel<ARGMAX>), dim3(g, M), dim3(MV_THREADS), 0, s, w, x, y,
                       idx, val, ws, N, static_cast<int>(K));
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_matvec(const uint8_t* w, const float* x, float* y, int64_t M, int64_t N,
                         int64_t K, hipStream_t s) {
  return launch_mv<false>(w, x, y, nullptr, nullptr, nullptr, M, N, K, s);
}

size_t lmhead_workspace_bytes(int64_t M) {
  return 256 + static_cast<size_t>(M) * AM_MAX_PARTIALS * 8;
}

hipError_t launch_lmhead_argmax(const uint8_t* w, const float* x, int32_t* out_idx, float* out_val,
                                int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t s) {
  return launch_mv<true>(w, x, nullptr, out_idx, out_val, workspace, M, N, K, s);
}

}  // namespace q4
