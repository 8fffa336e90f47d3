// Device-side helpers shared by the gfx950 kernels of the Q4_0 library.
//
// Q4_0 block (GGUF convention, the format named in section "Architecture" of
// "Implémentation en Rust du modèle Voxtral Mini 4B Realtime de Mistral pour
// l'exécuter dans le navigateur"): 18 bytes = binary16 scale d (little-endian)
// followed by qs[16]; weight j < 16 is qs[j] & 15, weight j + 16 is qs[j] >> 4,
// value (q - 8) * d.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

constexpr int QK = 32;           // weights per block
constexpr int BLOCK_BYTES = 18;  // bytes per block
constexpr int PAIR_BYTES = 36;   // two blocks: always dword aligned when the
                                 // first block's flat index is even

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// binary16 bit pattern (low 16 bits) -> float32, exact (subnormals kept).
__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  uint16_t b = static_cast<uint16_t>(bits);
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return static_cast<float>(h);
}

// Byte p of v as float; the backend selects v_cvt_f32_ubyte{p} for this.
template <int P>
__device__ __forceinline__ float ubyte_f(uint32_t v) {
  return static_cast<float>((v >> (8 * P)) & 0xFFu);
}

// Bytes [2..5] of the 8-byte window (lo, hi): funnel shift by 16 bits.
__device__ __forceinline__ uint32_t shift16(uint32_t hi, uint32_t lo) {
  return __builtin_amdgcn_alignbit(hi, lo, 16);
}

// sum_{t<4} (lo nibble of byte t of q - 8) * xl[t] + (hi nibble - 8) * xh[t]:
// the centred codes q - 8 (exact in float32), so the rounding of the sum is
// relative to sum |w x|.
__device__ __forceinline__ float nib_dot4_centred(uint32_t q, f32x4 xl, f32x4 xh, float acc) {
  uint32_t lo = q & 0x0F0F0F0Fu;
  uint32_t hi = (q >> 4) & 0x0F0F0F0Fu;
  // Keep the masked dwords opaque so each code costs one v_cvt_f32_ubyteN
  // rather than a bit-field extract plus a convert.
  asm("" : "+v"(lo));
  asm("" : "+v"(hi));
  acc = __builtin_fmaf(ubyte_f<0>(lo) - 8.f, xl.x, acc);
  acc = __builtin_fmaf(ubyte_f<1>(lo) - 8.f, xl.y, acc);
  acc = __builtin_fmaf(ubyte_f<2>(lo) - 8.f, xl.z, acc);
  acc = __builtin_fmaf(ubyte_f<3>(lo) - 8.f, xl.w, acc);
  acc = __builtin_fmaf(ubyte_f<0>(hi) - 8.f, xh.x, acc);
  acc = __builtin_fmaf(ubyte_f<1>(hi) - 8.f, xh.y, acc);
  acc = __builtin_fmaf(ubyte_f<2>(hi) - 8.f, xh.z, acc);
  acc = __builtin_fmaf(ubyte_f<3>(hi) - 8.f, xh.w, acc);
  return acc;
}

// Load block `f` (flat block index over the whole byte array) with 16-bit
// loads only: works for any block alignment.  d16 = scale bits, qs[4] = the
// 16 code bytes as little-endian dwords.
__device__ __forceinline__ void load_block_any(const uint8_t* __restrict__ base, int64_t f,
                                               uint32_t& d16, uint32_t qs[4]) {
  const uint16_t* p = reinterpret_cast<const uint16_t*>(base + f * BLOCK_BYTES);
  d16 = p[0];
#pragma unroll
  for (int t = 0; t < 4; ++t) qs[t] = static_cast<uint32_t>(p[1 + 2 * t]) | (static_cast<uint32_t>(p[2 + 2 * t]) << 16);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane of the
// row receives the same bits.  Each step adds a lane's partner from a
// symmetric pairing (swap within pairs, within quads, mirror within half
// rows, mirror within the row), so two partners add the same two values and
// get the same result.  The add order is the same in every row.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  return v;
}

}  // namespace q4
