// Q4_0 matrix-matrix product on the CDNA4 matrix cores: Y = X * deq(W)^T.
//
// Section "Architecture" of "Implémentation en Rust du modèle Voxtral Mini 4B
// Realtime de Mistral pour l'exécuter dans le navigateur": the audio encoder
// (width 1280) and the adapter after the 4x convolutional downsample run their
// projections over many frames at once, and the decoder's prompt prefix (38,
// 76 tokens: section "Correction du padding Q4") does the same for several
// tokens; these are dense contractions, so they go to v_mfma_f32_16x16x32_f16.
//
// Tiling: a 256-thread workgroup (4 waves, 2 x 2) owns a 128 x 128 tile of Y;
// each wave a 64 x 64 sub-tile = 4 x 4 MFMA tiles of 16 x 16, accumulated in
// float32 over K in steps of one Q4_0 block (32 = the MFMA's K).  Per step the
// workgroup converts X (float32 -> binary16, round to nearest even) and decodes
// the W block ((q - 8) * d computed in binary16: exact q - 8, one rounding of
// the product) into LDS, double-buffered, in the MFMA operand order, so every
// wave reads its fragments as contiguous 1 KiB rows of LDS.
//
// Operand order.  The MFMA sums over k, so any permutation of k applied to
// both operands gives the same products.  Lane l = i + 16 g (i < 16, g < 4)
// carries row/column i and the eight k values {4g..4g+3, 16+4g..16+4g+3} of
// the block: exactly the low and high nibbles of the four code bytes
// qs[4g..4g+3], so one dword of codes is one lane's operand.

#include "q4_device.h"
#include "q4_kernels.h"

namespace q4 {
namespace {

constexpr int MM_THREADS = 256;
constexpr int MM_BM = 128;
constexpr int MM_BN = 128;

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Decode the 8 codes of one qs dword into binary16 (q - 8) * d in operand order.
__device__ __forceinline__ f16x8 decode8_f16(uint32_t qs, uint32_t d16) {
  const uint32_t lo = qs & 0x0F0F0F0Fu;
  const uint32_t hi = (qs >> 4) & 0x0F0F0F0Fu;
  // v_perm: place a code in the low byte of each half with 0x64 above it,
  // i.e. the binary16 value 1024 + q; subtracting 1032 leaves q - 8 exactly.
  const uint32_t magic = 0x64646464u;
  const f16x2 off = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
  _Float16 dh;
  {
    const uint16_t b = static_cast<uint16_t>(d16);
    __builtin_memcpy(&dh, &b, 2);
  }
  const f16x2 dd = {dh, dh};
  f16x2 h0 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(magic, lo, 0x04010400u));
  f16x2 h1 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(magic, lo, 0x04030402u));
  f16x2 h2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(magic, hi, 0x04010400u));
  f16x2 h3 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(magic, hi, 0x04030402u));
  h0 = (h0 + off) * dd;
  h1 = (h1 + off) * dd;
  h2 = (h2 + off) * dd;
  h3 = (h3 + off) * dd;
  f16x8 r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

__device__ __forceinline__ f16x8 cvt8_f16(f32x4 a, f32x4 b) {
  f16x8 r;
  r[0] = static_cast<_Float16>(a.x); r[1] = static_cast<_Float16>(a.y);
  r[2] = static_cast<_Float16>(a.z); r[3] = static_cast<_Float16>(a.w);
  r[4] = static_cast<_Float16>(b.x); r[5] = static_cast<_Float16>(b.y);
  r[6] = static_cast<_Float16>(b.z); r[7] = static_cast<_Float16>(b.w);
  return r;
}

__global__ __launch_bounds__(MM_THREADS) void matmul_mfma_kernel(
    const uint8_t* __restrict__ W, const float* __restrict__ X, float* __restrict__ Y, int M, int N,
    int K) {
  __shared__ f16x8 As[2][MM_BM / 16][64];
  __shared__ f16x8 Bs[2][MM_BN / 16][64];

  const int nb = K / QK;
  const int m0 = blockIdx.y * MM_BM;
  const int n0 = blockIdx.x * MM_BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Loader items: it = tid + 256 u (u = 0, 1): row r = it >> 2 (0..127), group g = it & 3.
  f32x4 a_lo[2], a_hi[2];
  uint32_t b_d[2], b_q[2];

  auto load_stage = [&](int kb) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int it = tid + MM_THREADS * u;
      const int r = it >> 2, g = it & 3;
      const int m = m0 + r;
      if (m < M) {
        const float* xr = X + static_cast<int64_t>(m) * K + kb * QK;
        a_lo[u] = *reinterpret_cast<const f32x4*>(xr + 4 * g);
        a_hi[u] = *reinterpret_cast<const f32x4*>(xr + 16 + 4 * g);
      } else {
        a_lo[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        a_hi[u] = a_lo[u];
      }
      const int n = n0 + r;
      if (n < N) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(
            W + (static_cast<int64_t>(n) * nb + kb) * BLOCK_BYTES);
        b_d[u] = p[0];
        b_q[u] = static_cast<uint32_t>(p[1 + 2 * g]) | (static_cast<uint32_t>(p[2 + 2 * g]) << 16);
      } else {
        b_d[u] = 0u;  // scale 0: decodes to zeros
        b_q[u] = 0x88888888u;
      }
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int it = tid + MM_THREADS * u;
      const int r = it >> 2, g = it & 3;
      As[buf][r >> 4][(r & 15) + 16 * g] = cvt8_f16(a_lo[u], a_hi[u]);
      Bs[buf][r >> 4][(r & 15) + 16 * g] = decode8_f16(b_q[u], b_d[u]);
    }
  };

  f32x4v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) acc[i][jn] = f32x4v{0.f, 0.f, 0.f, 0.f};

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kb = 0; kb < nb; ++kb) {
    const int cur = kb & 1;
    const bool more = kb + 1 < nb;
    if (more) load_stage(kb + 1);
    f16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = As[cur][wm * 4 + i][lane];
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) b[jn] = Bs[cur][wn * 4 + jn][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jn = 0; jn < 4; ++jn)
        acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[jn], acc[i][jn], 0, 0, 0);
    if (more) store_stage(cur ^ 1);
    __syncthreads();
  }

  // 16 x 16 accumulator layout: lane l holds column l % 16, rows 4 (l / 16) + v.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
      const int col = n0 + wn * 64 + jn * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + v;
        if (row < M) Y[static_cast<int64_t>(row) * N + col] = acc[i][jn][v];
      }
    }
  }
}

}  // namespace

hipError_t launch_matmul(const uint8_t* w, const float* x, float* y, int64_t M, int64_t N,
                         int64_t K, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((N + MM_BN - 1) / MM_BN),
                  static_cast<unsigned>((M + MM_BM - 1) / MM_BM));
  hipLaunchKernelGGL(matmul_mfma_kernel, grid, dim3(MM_THREADS), 0, s, w, x, y,
                     static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
  return hipGetLastError();
}

}  // namespace q4
