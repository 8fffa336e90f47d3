// Token-embedding gather-decode and the device-side Q4_0 encoder.
//
// Section "Solutions techniques pour l'exécution dans le navigateur", item 3,
// of "Implémentation en Rust du modèle Voxtral Mini 4B Realtime de Mistral
// pour l'exécuter dans le navigateur": the 1.5 GiB embedding table stays in Q4
// on the GPU and rows are looked up by token id.  Here the lookup itself runs
// on the GPU: one thread decodes one 32-weight block of one requested row.
//
// The encoder implements the GGUF Q4_0 rule (the format of section
// "Architecture"): per block, m = first element of largest |x|, d = m / -8 in
// float32 stored as binary16 (round to nearest even), codes decided in float64
// against the stored scale with half-up rounding, clamped to [0, 15].  One
// thread per block.

#include "q4_device.h"
#include "q4_kernels.h"

namespace q4 {
namespace {

constexpr int EQ_THREADS = 128;

__global__ __launch_bounds__(EQ_THREADS) void embed_kernel(const uint8_t* __restrict__ T,
                                                           const int32_t* __restrict__ ids,
                                                           float* __restrict__ out, int64_t M,
                                                           int64_t N, int K) {
  const int nb = K / QK;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * EQ_THREADS + threadIdx.x;
  if (t >= M * nb) return;
  const int64_t i = t / nb;
  const int b = static_cast<int>(t - i * nb);
  const int64_t id = ids[i];
  f32x4* dst = reinterpret_cast<f32x4*>(out + i * K + static_cast<int64_t>(b) * QK);
  if (id < 0 || id >= N) {
#pragma unroll
    for (int u = 0; u < 8; ++u) dst[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  uint32_t d16, qs[4];
  load_block_any(T, id * nb + b, d16, qs);
  const float d = half_bits_to_float(d16);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t lo = qs[u] & 0x0F0F0F0Fu;
    const uint32_t hi = (qs[u] >> 4) & 0x0F0F0F0Fu;
    dst[u] = f32x4{(ubyte_f<0>(lo) - 8.f) * d, (ubyte_f<1>(lo) - 8.f) * d,
                   (ubyte_f<2>(lo) - 8.f) * d, (ubyte_f<3>(lo) - 8.f) * d};
    dst[4 + u] = f32x4{(ubyte_f<0>(hi) - 8.f) * d, (ubyte_f<1>(hi) - 8.f) * d,
                       (ubyte_f<2>(hi) - 8.f) * d, (ubyte_f<3>(hi) - 8.f) * d};
  }
}

__global__ __launch_bounds__(EQ_THREADS) void quantize_kernel(const float* __restrict__ w,
                                                              uint8_t* __restrict__ out,
                                                              int64_t nblocks,
                                                              int32_t* __restrict__ flag) {
  const int64_t f = static_cast<int64_t>(blockIdx.x) * EQ_THREADS + threadIdx.x;
  if (f >= nblocks) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(w + f * QK);
  float v[QK];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const f32x4 a = src[u];
    v[4 * u] = a.x; v[4 * u + 1] = a.y; v[4 * u + 2] = a.z; v[4 * u + 3] = a.w;
  }
  // first element of largest magnitude, sign kept
  bool bad = false;
  float amax = -1.f, m = 0.f;
#pragma unroll
  for (int i = 0; i < QK; ++i) {
    const float a = __builtin_fabsf(v[i]);
    bad |= !(a <= 3.402823466e38f);  // inf or NaN
    if (a > amax) { amax = a; m = v[i]; }
  }
  float d = m / -8.0f;
  // Keep the division and the binary16 conversion separate: fused into one
  // mixed-precision FMA with a +0 addend, m = +0 would give +0 instead of -0.
  asm volatile("" : "+v"(d));
  const _Float16 dh = static_cast<_Float16>(d);
  uint16_t dbits;
  __builtin_memcpy(&dbits, &dh, 2);
  bad |= (dbits & 0x7C00u) == 0x7C00u;
  uint32_t q[QK];
  if ((dbits & 0x7FFFu) == 0u) {
#pragma unroll
    for (int i = 0; i < QK; ++i) q[i] = 8u;
  } else {
    const double dd = static_cast<double>(dh);
#pragma unroll
    for (int i = 0; i < QK; ++i) {
      const double t = static_cast<double>(v[i]) / dd;
      const double fl = __builtin_floor(t);
      double r = fl + ((t - fl) >= 0.5 ? 1.0 : 0.0) + 8.0;
      r = r < 0.0 ? 0.0 : (r > 15.0 ? 15.0 : r);
      q[i] = static_cast<uint32_t>(r);
    }
  }
  uint16_t* o = reinterpret_cast<uint16_t*>(out + f * BLOCK_BYTES);
  o[0] = dbits;
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const uint32_t b0 = q[2 * h] | (q[2 * h + 16] << 4);
    const uint32_t b1 = q[2 * h + 1] | (q[2 * h + 17] << 4);
    o[1 + h] = static_cast<uint16_t>(b0 | (b1 << 8));
  }
  if (bad && flag) *flag = 1;
}

}  // namespace

hipError_t launch_embed(const uint8_t* table, const int32_t* ids, float* out, int64_t M,
                        int64_t N, int64_t K, hipStream_t s) {
  const int64_t items = M * (K / QK);
  const unsigned grid = static_cast<unsigned>((items + EQ_THREADS - 1) / EQ_THREADS);
  hipLaunchKernelGGL(embed_kernel, dim3(grid), dim3(EQ_THREADS), 0, s, table, ids, out, M, N,
                     static_cast<int>(K));
  return hipGetLastError();
}

hipError_t launch_quantize(const float* w, uint8_t* out, int64_t N, int64_t K, int32_t* flag,
                           hipStream_t s) {
  const int64_t nblocks = N * (K / QK);
  const unsigned grid = static_cast<unsigned>((nblocks + EQ_THREADS - 1) / EQ_THREADS);
  hipLaunchKernelGGL(quantize_kernel, dim3(grid), dim3(EQ_THREADS), 0, s, w, out, nblocks, flag);
  return hipGetLastError();
}

}  // namespace q4
