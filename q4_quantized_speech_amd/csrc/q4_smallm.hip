// Q4_0 product for up to four rows of x (several decode streams at once),
// reading every weight byte once, with the accuracy of an f32 dot product.
//
// Section "Architecture" of "Implémentation en Rust du modèle Voxtral Mini 4B
// Realtime de Mistral pour l'exécuter dans le navigateur" runs every decoder
// projection on Q4_0 weights.  With a few rows of x the product is still an
// HBM stream; one FMA per weight and row would make the vector ALUs the limit
// past two rows, so the multiply goes to the matrix cores:
//  * the weights enter v_mfma_f32_16x16x32_f16 as q - 8 (exact in binary16),
//    one MFMA per 32-weight block, and each block's scale d multiplies the
//    MFMA result in f32 (no rounding of (q - 8) * d to binary16);
//  * x is split into two binary16 parts, x = hi + lo with lo = x - hi, after
//    scaling each row's 256-value chunk by the power of two that puts its
//    largest magnitude in [2^14, 2^15) (range safe, undone exactly after the
//    chunk): two MFMAs per block carry about 22 significant bits of x;
//  * that holds for the values of a chunk within 2^20 of its largest: they
//    scale to at least 2^-6, where the two parts keep a relative error below
//    2^-19.  A chunk (of one row of x) whose nonzero magnitudes span more
//    than 2^20, or whose largest is 2^124 or more (or not finite), would lose
//    its small values to binary16 subnormals or overflow; it is "wide": its
//    binary16 operands are zero, and the waves add its products with float32
//    FMAs of the centred codes (q - 8) against the float32 x, as q4_matvec
//    does.  Normal activations rarely have one (a value below 2^-20 of the
//    chunk's largest), so the float32 path costs nothing in practice;
//  * a workgroup owns 64 rows of W (four waves of 16 rows) and a range of K,
//    taken in segments of four 256-value chunks; x of a segment is staged in
//    LDS in the MFMA operand layout (wave w stages chunk w), shared by the
//    four waves;
//  * each lane loads one contiguous 36-byte block pair of its row (lanes
//    16 g + n: row n, pair g of a chunk); a 4 x 4 transpose across the four
//    lane rows (v_permlane32_swap, v_permlane16_swap) gives lane (n, g) the
//    code dword g of every block of the chunk, the MFMA operand layout;
//  * a segment's four chunks of weights are requested together, after its x;
//    while one segment is computed the next one's x and, chunk by chunk, its
//    weights are in flight.  K ranges of several workgroups (a K split) are
//    added by the fold kernel in a fixed order: results are deterministic.

#include <atomic>

#include "q4_device.h"
#include "q4_kernels.h"

namespace q4 {
namespace {

constexpr int SM_THREADS = 256;  // four waves
constexpr int SM_ROWS = 64;      // rows of W per workgroup
constexpr int SM_SEGC = 4;       // chunks (256 values of K each) per x segment; one per wave
constexpr int SM_SEGB = SM_SEGC * 8;  // blocks per segment
constexpr int SM_MAX_M = 4;      // rows of x (more go to the binary16 skinny kernel)

typedef float f32x4m __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sm_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// Row g (lanes 16 g .. 16 g + 15) of r[t] holds X[g][t]; afterwards row g of
// r[p] holds X[p][g].
__device__ __forceinline__ void transpose4(uint32_t (&r)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  r[0] = c[0];
  r[1] = c[1];
  r[2] = d[0];
  r[3] = d[1];
}

// The 8 codes of one qs dword as binary16 q - 8 (exact), in the order
// [byte 0..3 low nibbles, byte 0..3 high nibbles] = elements
// {4g..4g+3, 16+4g..16+4g+3} of the block for code dword g.
__device__ __forceinline__ f16x8 decode8_q(uint32_t qs) {
  const uint32_t lo = qs & 0x0F0F0F0Fu;
  const uint32_t hi = (qs >> 4) & 0x0F0F0F0Fu;
  // v_perm puts each code under the byte 0x64: the binary16 1024 + q.
  const uint32_t magic = 0x64646464u;
  const f16x2 off = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
  const f16x2 h0 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(magic, lo, 0x04010400u)) + off;
  const f16x2 h1 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(magic, lo, 0x04030402u)) + off;
  const f16x2 h2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(magic, hi, 0x04010400u)) + off;
  const f16x2 h3 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(magic, hi, 0x04030402u)) + off;
  f16x8 r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

// Largest of a non-negative value over the wave, in every lane: DPP within
// each row of 16 lanes, then the two permlane swaps across rows.
__device__ __forceinline__ float wave_max_nonneg(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp_f32<0x128>(v));  // row_ror:8
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Smallest of a non-negative value over the wave, in every lane (the same
// pattern of exchanges as wave_max_nonneg).
__device__ __forceinline__ float wave_min_nonneg(float v) {
  v = fminf(v, dpp_f32<0xB1>(v));
  v = fminf(v, dpp_f32<0x4E>(v));
  v = fminf(v, dpp_f32<0x124>(v));
  v = fminf(v, dpp_f32<0x128>(v));
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fminf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Power-of-two exponent that scales a row whose largest magnitude has the
// float bits `mbits` (non-negative) into [2^14, 2^15); clamped so that the
// scale and its inverse stay normal floats.
__device__ __forceinline__ int scale_exp(uint32_t mbits) {
  const int eb = static_cast<int>(mbits >> 23);  // biased exponent (255: inf or NaN)
  int s = 141 - eb;
  s = s < -110 ? -110 : s;
  return s > 110 ? 110 : s;
}
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float(static_cast<uint32_t>(e + 127) << 23); }

// grid = tiles * splits; workgroup b: row tile b % tiles, K split b / tiles
// (pairs [split * pps, min(nbp, (split + 1) * pps)), pps a multiple of 4).
// MR >= M rows of x are loaded (a multiple of 4).  splits == 1: Y[m][n]
// directly; else partials P[split][m][n].
template <int MR>
__global__ __launch_bounds__(SM_THREADS) void matmul_small_kernel(
    const uint8_t* __restrict__ W, const float* __restrict__ X, float* __restrict__ Y,
    float* __restrict__ P, int M, int N, int K, int tiles, int pps) {
  // x operands [block][group g][row m]: entry m < MR is the hi (lo) operand
  // of lane (m, g); entry MR stays zero and serves the lanes of rows >= MR.
  __shared__ f16x8 xh[SM_SEGB][4][MR + 1];
  __shared__ f16x8 xl[SM_SEGB][4][MR + 1];
  __shared__ f32x4m usc[SM_SEGC][4];  // [chunk][row / 4]: 2^-scale of each row of x
  // wide chunks: the float32 x of each (chunk, row), and per chunk a bit
  // mask of the rows whose chunk is wide (0: all rows on the matrix cores)
  __shared__ __attribute__((aligned(16))) float xf[SM_SEGC][MR][256];
  __shared__ uint32_t wflag[SM_SEGC];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int xm = n < MR ? n : MR;  // this lane's operand entry (row n of x, or the zero entry)
  const int tile = static_cast<int>(blockIdx.x) % tiles;
  const int split = static_cast<int>(blockIdx.x) / tiles;
  const int nbp = K >> 6;
  const int p_begin = split * pps;
  const int p_end = min(nbp, p_begin + pps);
  const int64_t rb = static_cast<int64_t>(nbp) * PAIR_BYTES;
  const int64_t row_base = static_cast<int64_t>(tile) * SM_ROWS;
  const int rows_valid = static_cast<int>(min<int64_t>(SM_ROWS, N - row_base));
  const int records = static_cast<int>(rows_valid * rb);
  const __amdgpu_buffer_rsrc_t rs = sm_rsrc(W + row_base * rb, records);
  const int rowoff = static_cast<int>((wave * 16 + n) * rb);
  const int xrec = M * K * 4;
  const __amdgpu_buffer_rsrc_t xrs = sm_rsrc(X, xrec);

  // Pair 4 c + g of this lane's row; pairs past the K range (and rows past
  // N) read as zeros, with no memory traffic: codes 0 with scale 0 against x
  // staged as 0.
  auto load = [&](int c, uint32_t (&D)[9]) {
    const int pc = 4 * c + g;
    const int vo = pc < p_end ? rowoff + pc * PAIR_BYTES : records;
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 0, 0));
    const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 16, 0));
    D[0] = a.x; D[1] = a.y; D[2] = a.z; D[3] = a.w;
    D[4] = b.x; D[5] = b.y; D[6] = b.z; D[7] = b.w;
    D[8] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo, 32, 0);
  };

  // x of a segment (chunks [c0, c0 + 4)): wave w takes chunk c0 + w, lane l
  // the float4 l of that chunk in every row.  Rows past M and values past the
  // K range read as zeros (no traffic); every load is issued, so the memory
  // counter waits stay exact.
  const int c_begin = p_begin >> 2, c_end = (p_end + 3) >> 2;
  auto stage_load = [&](int c0, f32x4m (&v)[MR]) {
    const int k = ((c0 + wave) << 8) + 4 * lane;
    const bool kv = k < (p_end << 6);
#pragma unroll
    for (int u = 0; u < MR; ++u) {
      const int vo = kv && u < M ? 4 * (u * K + k) : xrec;  // the whole offset in the range check
      v[u] = __builtin_bit_cast(f32x4m, __builtin_amdgcn_raw_buffer_load_b128(xrs, vo, 0, 0));
    }
  };
  // Each row's chunk is scaled by the power of two that puts its largest
  // magnitude in [2^14, 2^15) (a wave maximum: one chunk is one wave), split
  // into hi/lo binary16 and stored in operand order; a wide chunk (see the
  // header) stores zero operands and its float32 values instead.
  auto stage_store = [&](const f32x4m (&v)[MR]) {
    const int k = 4 * lane, blk = wave * 8 + (k >> 5), e = k & 31;
    const int gg = (e & 15) >> 2, half = e >> 4;  // operand group, low/high nibble half
    uint32_t wmask = 0;
#pragma unroll
    for (int u = 0; u < MR; ++u) {
      if (u < M) {
        const f32x4m av = {fabsf(v[u].x), fabsf(v[u].y), fabsf(v[u].z), fabsf(v[u].w)};
        const float a = fmaxf(fmaxf(av.x, av.y), fmaxf(av.z, av.w));
        // smallest nonzero magnitude (+inf when all four are zero; NaN never
        // counts, in neither reduction)
        float z = __builtin_inff();
        z = av.x > 0.f ? fminf(z, av.x) : z;
        z = av.y > 0.f ? fminf(z, av.y) : z;
        z = av.z > 0.f ? fminf(z, av.z) : z;
        z = av.w > 0.f ? fminf(z, av.w) : z;
        const float cmax = wave_max_nonneg(a);
        const float cmin = wave_min_nonneg(z);
        // the same in every lane of the wave (both reductions end in all lanes)
        const bool wide = !(cmax < 0x1p124f) || cmin < cmax * 0x1p-20f;
        const int se = scale_exp(__float_as_uint(cmax));
        uint32_t* ph = reinterpret_cast<uint32_t*>(&xh[blk][gg][u]) + 2 * half;
        uint32_t* pl = reinterpret_cast<uint32_t*>(&xl[blk][gg][u]) + 2 * half;
        if (wide) {
          ph[0] = ph[1] = pl[0] = pl[1] = 0u;
          *reinterpret_cast<f32x4m*>(&xf[wave][u][k]) = v[u];
          wmask |= 1u << u;
        } else {
          const f32x4m xv = v[u] * exp2i(se);
          const f16x2 h01 = {static_cast<_Float16>(xv.x), static_cast<_Float16>(xv.y)};
          const f16x2 h23 = {static_cast<_Float16>(xv.z), static_cast<_Float16>(xv.w)};
          const f16x2 l01 = {static_cast<_Float16>(xv.x - static_cast<float>(h01[0])),
                             static_cast<_Float16>(xv.y - static_cast<float>(h01[1]))};
          const f16x2 l23 = {static_cast<_Float16>(xv.z - static_cast<float>(h23[0])),
                             static_cast<_Float16>(xv.w - static_cast<float>(h23[1]))};
          ph[0] = __builtin_bit_cast(uint32_t, h01);
          ph[1] = __builtin_bit_cast(uint32_t, h23);
          pl[0] = __builtin_bit_cast(uint32_t, l01);
          pl[1] = __builtin_bit_cast(uint32_t, l23);
        }
        if (lane == 0) usc[wave][u >> 2][u & 3] = exp2i(-se);
      }
    }
    if (lane == 0) wflag[wave] = wmask;
  };

  // One chunk (4 pairs = 8 blocks) of this wave's 16 rows; cs = chunk index
  // within the segment.  Adds to acc[v] (row m = 4 g + v of x, W row n).
  auto compute = [&](const uint32_t (&D)[9], int cs, f32x4m& acc) {
    uint32_t E[4], O[4], S[4];
    E[0] = shift16(D[1], D[0]);
    E[1] = shift16(D[2], D[1]);
    E[2] = shift16(D[3], D[2]);
    E[3] = shift16(D[4], D[3]);
    O[0] = D[5]; O[1] = D[6]; O[2] = D[7]; O[3] = D[8];
    const uint32_t dd = (D[0] & 0xFFFFu) | (D[4] & 0xFFFF0000u);  // scales of the pair's blocks
    S[0] = dd; S[1] = dd; S[2] = dd; S[3] = dd;
    transpose4(E);
    transpose4(O);
    transpose4(S);  // S[p] = scales of pair p of this row (all four lane rows)
    f32x4m cacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f16x8 b = decode8_q(h ? O[p] : E[p]);
        const int blk = cs * 8 + 2 * p + h;
        f32x4m c = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh[blk][g][xm], b, f32x4m{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[blk][g][xm], b, c, 0, 0, 0);
        const float d = half_bits_to_float(h ? (S[p] >> 16) : (S[p] & 0xFFFFu));
        cacc.x = __builtin_fmaf(d, c.x, cacc.x);
        cacc.y = __builtin_fmaf(d, c.y, cacc.y);
        cacc.z = __builtin_fmaf(d, c.z, cacc.z);
        cacc.w = __builtin_fmaf(d, c.w, cacc.w);
      }
    }
    const f32x4m u = usc[cs][g];
    acc.x = __builtin_fmaf(cacc.x, u.x, acc.x);
    acc.y = __builtin_fmaf(cacc.y, u.y, acc.y);
    acc.z = __builtin_fmaf(cacc.z, u.z, acc.z);
    acc.w = __builtin_fmaf(cacc.w, u.w, acc.w);
    // Wide chunks (rare; the mask is the same for the whole workgroup): the
    // lane's 8 weights of each block against the float32 x, centred codes,
    // the block scale per block; the four lane groups' sums are added in a
    // fixed order and land in every lane.  Lane group 0 holds rows 0..3 of
    // x in acc's components; the other groups' components are rows past 4,
    // never stored, so the sum is added in every lane without a branch.
    const uint32_t wm = wflag[cs];
    if (wm != 0u) {
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        if ((wm >> r) & 1u) {
          const float* xr = &xf[cs][r][0];
          float part = 0.f;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int b32 = 32 * (2 * p + h);
              const f32x4m xlo = *reinterpret_cast<const f32x4m*>(xr + b32 + 4 * g);
              const f32x4m xhi = *reinterpret_cast<const f32x4m*>(xr + b32 + 16 + 4 * g);
              const float d = half_bits_to_float(h ? (S[p] >> 16) : (S[p] & 0xFFFFu));
              part = __builtin_fmaf(d, nib_dot4_centred(h ? O[p] : E[p], xlo, xhi, 0.f), part);
            }
          }
          part += __shfl_xor(part, 16);
          part += __shfl_xor(part, 32);
          acc[r] += part;
        }
      }
    }
  };

  {  // operand entries of rows >= M (and the zero entry) stay zero throughout
    const f16x8 z = {};
    for (int e = tid; e < SM_SEGB * 4 * (MR + 1); e += SM_THREADS) {
      const int m = e % (MR + 1), bg = e / (MR + 1);
      if (m >= M) {
        xh[bg >> 2][bg & 3][m] = z;
        xl[bg >> 2][bg & 3][m] = z;
      }
    }
  }

  // x of a segment is requested first, then the segment's weights; while a
  // segment is computed, the next segment's x and (chunk by chunk, into the
  // registers just freed) its weights are in flight.
  f32x4m acc = {0.f, 0.f, 0.f, 0.f};
  uint32_t d0[9], d1[9], d2[9], d3[9];
  f32x4m v[MR];
  int s0 = c_begin;
  stage_load(s0, v);
  load(s0, d0);
  load(s0 + 1, d1);
  load(s0 + 2, d2);
  load(s0 + 3, d3);
  for (;;) {
    stage_store(v);
    __syncthreads();
    const int s1 = s0 + SM_SEGC;
    stage_load(s1, v);
    compute(d0, 0, acc);
    load(s1, d0);
    if (s0 + 1 < c_end) compute(d1, 1, acc);
    load(s1 + 1, d1);
    if (s0 + 2 < c_end) compute(d2, 2, acc);
    load(s1 + 2, d2);
    if (s0 + 3 < c_end) compute(d3, 3, acc);
    load(s1 + 3, d3);
    if (s1 >= c_end) break;
    __syncthreads();  // every wave is done with this segment's x
    s0 = s1;
  }

  const int64_t row = row_base + wave * 16 + n;
  if (row < N) {
    float* out = P ? P + static_cast<int64_t>(split) * M * N : Y;
    const float vals[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      if (m < M) out[static_cast<int64_t>(m) * N + row] = vals[v];
    }
  }
}

// ---------------------------------------------------------------------------
// Two to 48 rows of x (a short prompt prefix, a few decode streams at
// once): the product is still an HBM stream, and one 16 x 16 x 32 MFMA per
// weight block and 16 rows of x carries them, so the work per weight is
// nearly that of a single row.  The kernel has the matvec's shape: a
// persistent workgroup of KS waves splits K (wave w owns C consecutive
// 256-value chunks), holds its x in registers for the whole kernel and
// streams 16 weight rows per pass:
//  * x is converted once per workgroup to binary16 (round to nearest even)
//    in the MFMA operand order (lane (m, g): row m of a 16-row tile of x,
//    code group g), MT tiles of 16 rows; for two to four rows (HL) as two
//    binary16 parts in one tile, described below;
//  * lane (n, g) loads the contiguous 36-byte pair g of weight row n of each
//    chunk (at one chunk per wave two passes in flight in two register
//    sets, at two a chunk's next load issued as soon as it is computed);
//    the 4 x 4 lane transpose of the small-M kernel gives it code dword g
//    of every block;
//  * with one tile of x the codes enter the matrix cores exactly (q - 8),
//    one MFMA per block, and the block scale d multiplies the MFMA result in
//    float32; with two or three tiles (q - 8) d rounded once to binary16 is
//    accumulated in the MFMA (the float32 products would not fit in the
//    registers);
//  * the KS waves' partial 16 x 16 tiles are added in LDS in wave order
//    (deterministic), one barrier per pass, and written to Y.
// No K split across workgroups, so no partial sums and no second launch.
constexpr int MS_MAX_MT = 3;   // tiles of 16 rows of x
constexpr int MS_MAX_WAVES = 16;

// HL (two to four rows of x, the q4_matvec bound): x is carried as two
// binary16 parts, hi = RN(x s) and lo = RN(x s - hi), with s the power of two
// that puts the largest magnitude of the row's 256-value chunk in
// [2^14, 2^15) (undone in float32 after the chunk): hi in rows 0-3 of the
// tile, lo in rows 4-7, so one MFMA per block carries both; a chunk whose
// nonzero magnitudes span more than 2^20 (or whose largest reaches 2^124, or
// is not finite) is "wide": its operands are zero and its products are added
// with float32 FMAs of the centred codes against x read again from memory,
// the rule and the arithmetic of the small-M kernel.
template <int C, int MT, bool HL>
__global__ __launch_bounds__(C == 1 && MT == 1 ? 1024 : 768) void matmul_stream16_kernel(
    const uint8_t* __restrict__ W, const float* __restrict__ X, float* __restrict__ Y, int M,
    int N, int K) {
  static_assert(MT >= 1 && MT <= MS_MAX_MT && (C == 1 || MT == 1), "registers: see the host side");
  static_assert(!HL || MT == 1, "two-part x: one tile");
  // x staging (one 8 KB tile per wave, in operand order), then, after a
  // barrier, the same memory holds the passes' partial tiles
  __shared__ f16x8 xst[MS_MAX_WAVES][512];
  f32x4m (*red)[MT][MS_MAX_WAVES][64] =
      reinterpret_cast<f32x4m (*)[MT][MS_MAX_WAVES][64]>(&xst[0][0]);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ks = static_cast<int>(blockDim.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int nbp = K >> 6;
  const int rb = nbp * PAIR_BYTES;  // K <= 6144: at most 3456
  const int units = (N + 15) >> 4;
  // a contiguous, balanced range of 16-row units per workgroup
  const int nwg = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
  const int q = units / nwg, rem = units % nwg;
  const int u_begin = b * q + min(b, rem);
  const int npass = q + (b < rem ? 1 : 0);

  // x operands of this wave's chunks, filled below once the first weights
  // are requested (rows past M and values past K: zero)
  f16x8 xa[C][MT][8];
  // HL: per chunk, 2^-s of each row of x and the mask of its wide rows
  // (the same in every lane of the wave)
  float xu[C][4];
  uint32_t xwide[C];
  const int xrec = M * K * 4;  // M <= 48, K <= 6144
  const __amdgpu_buffer_rsrc_t xrs = sm_rsrc(X, xrec);
  // Pair g of chunk j of weight row n of pass `pass`; rows past N, pairs past
  // K and passes past this workgroup's range read as zeros, with no traffic.
  auto load = [&](int pass, int j, uint32_t (&D)[9]) {
    const int64_t row_base = static_cast<int64_t>(u_begin + pass) * 16;
    const int rows_valid =
        pass < npass ? static_cast<int>(min<int64_t>(16, static_cast<int64_t>(N) - row_base)) : 0;
    const int records = rows_valid * rb;
    const __amdgpu_buffer_rsrc_t rs = sm_rsrc(W + (pass < npass ? row_base : 0) * rb, records);
    const int pc = 4 * (wave * C + j) + g;
    const int vo = (n < rows_valid && pc < nbp) ? n * rb + pc * PAIR_BYTES : records;
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 0, 0));
    const u32x4 c = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, vo, 16, 0));
    D[0] = a.x; D[1] = a.y; D[2] = a.z; D[3] = a.w;
    D[4] = c.x; D[5] = c.y; D[6] = c.z; D[7] = c.w;
    D[8] = __builtin_amdgcn_raw_buffer_load_b32(rs, vo, 32, 0);
  };

  // Chunk j of a pass into this wave's partial tiles (tile t: rows
  // m = 16 t + 4 g + v of x, weight row n).
  auto compute = [&](int j, const uint32_t (&D)[9], f32x4m (&acc)[MT]) {
    uint32_t E[4], O[4], S[4];
    E[0] = shift16(D[1], D[0]);
    E[1] = shift16(D[2], D[1]);
    E[2] = shift16(D[3], D[2]);
    E[3] = shift16(D[4], D[3]);
    O[0] = D[5]; O[1] = D[6]; O[2] = D[7]; O[3] = D[8];
    const uint32_t dd = (D[0] & 0xFFFFu) | (D[4] & 0xFFFF0000u);
    S[0] = dd; S[1] = dd; S[2] = dd; S[3] = dd;
    transpose4(E);
    transpose4(O);
    transpose4(S);  // S[p] = scales of pair p of this row
    f32x4m cacc = {0.f, 0.f, 0.f, 0.f};  // one tile, exact weights: this chunk's sum
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t dbits = h ? (S[p] >> 16) : (S[p] & 0xFFFFu);
        if constexpr (MT == 1) {
          // exact weights: q - 8 into the MFMA, d applied to its result
          const f16x8 bw = decode8_q(h ? O[p] : E[p]);
          const float d = half_bits_to_float(dbits);
          const f32x4m c = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              xa[j][0][2 * p + h], bw, f32x4m{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          cacc.x = __builtin_fmaf(d, c.x, cacc.x);
          cacc.y = __builtin_fmaf(d, c.y, cacc.y);
          cacc.z = __builtin_fmaf(d, c.z, cacc.z);
          cacc.w = __builtin_fmaf(d, c.w, cacc.w);
        } else {
          // two or three tiles of x: (q - 8) d rounded once to binary16 (as
          // on the skinny and wide routes) and accumulated in the MFMA; the
          // exact form's float32 products would not fit in the registers
          const _Float16 dh = __builtin_bit_cast(_Float16, static_cast<uint16_t>(dbits));
          const f16x8 bw = decode8_q(h ? O[p] : E[p]) * dh;
#pragma unroll
          for (int t = 0; t < MT; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[j][t][2 * p + h], bw, acc[t], 0, 0, 0);
        }
      }
    }
    if constexpr (MT == 1 && !HL) {
      acc[0] += cacc;
    } else if constexpr (HL) {
      // lane groups 0 and 1 hold the hi and lo sums of row v of x: undo the
      // chunk's scaling of that row (groups 2 and 3 hold zero rows)
      acc[0].x = __builtin_fmaf(cacc.x, xu[j][0], acc[0].x);
      acc[0].y = __builtin_fmaf(cacc.y, xu[j][1], acc[0].y);
      acc[0].z = __builtin_fmaf(cacc.z, xu[j][2], acc[0].z);
      acc[0].w = __builtin_fmaf(cacc.w, xu[j][3], acc[0].w);
      // wide rows of this chunk (rare; the mask is the same for the whole
      // wave): the lane's 8 codes of each block against the float32 x,
      // centred codes, the block scale per block; the four lane groups' sums
      // are added in a fixed order and land in lane group 0 (the hi rows)
      if (xwide[j] != 0u) {
        const int kb = (wave * C + j) << 8;
        // one row at a time, not unrolled (the rare path must not raise the
        // register count of the common one)
#pragma unroll 1
        for (int r = 0; r < 4; ++r) {
          if ((xwide[j] >> r) & 1u) {
            float part = 0.f;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const int k0 = kb + 64 * p + 32 * h + 4 * g;
                const int vo = k0 < K ? 4 * (r * K + k0) : xrec;
                const f32x4 xl = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, vo, 0, 0));
                const f32x4 xh = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, vo, 64, 0));
                const float d = half_bits_to_float(h ? (S[p] >> 16) : (S[p] & 0xFFFFu));
                part = __builtin_fmaf(d, nib_dot4_centred(h ? O[p] : E[p], xl, xh, 0.f), part);
                // one block at a time: the rare path must not raise the
                // register count of the common one by hoisting its loads
                __builtin_amdgcn_sched_barrier(0);
              }
            }
            part += __shfl_xor(part, 16);
            part += __shfl_xor(part, 32);
            const float add = g == 0 ? part : 0.f;
            acc[0].x += r == 0 ? add : 0.f;
            acc[0].y += r == 1 ? add : 0.f;
            acc[0].z += r == 2 ? add : 0.f;
            acc[0].w += r == 3 ? add : 0.f;
          }
        }
      }
    }
  };

  // The waves' partial tiles of a pass, added in wave order, to Y's 16
  // columns of the pass.
  auto finish = [&](int pass, const f32x4m (&acc)[MT]) {
    const int par = pass & 1;
#pragma unroll
    for (int t = 0; t < MT; ++t) red[par][t][wave][lane] = acc[t];
    __syncthreads();
    if constexpr (HL) {
      // output (m, nn), m < 4: the hi sum (lane nn) and the lo sum (lane
      // nn + 16), component m, each over the waves in wave order
      for (int o = tid; o < 64; o += 64 * ks) {
        const int m = o >> 4, nn = o & 15;
        const float* sh = reinterpret_cast<const float*>(&red[par][0][0][nn]) + m;
        const float* sl = reinterpret_cast<const float*>(&red[par][0][0][nn + 16]) + m;
        float hi = 0.f, lo = 0.f;
        for (int w = 0; w < ks; ++w) {
          hi += sh[w * 64 * 4];
          lo += sl[w * 64 * 4];
        }
        const int64_t col = static_cast<int64_t>(u_begin + pass) * 16 + nn;
        if (m < M && col < N) Y[static_cast<int64_t>(m) * N + col] = hi + lo;
      }
      return;
    }
    // output (m, nn): row m = 16 t + mm of x, weight row nn of the pass; its
    // partials sit in tile t, lane nn + 16 (mm / 4), component mm % 4, of
    // every wave (workgroups of fewer threads than outputs take them in turns)
    for (int o = tid; o < 256 * MT; o += 64 * ks) {
      const int t = o >> 8, mm = (o >> 4) & 15, nn = o & 15;
      const float* src =
          reinterpret_cast<const float*>(&red[par][t][0][nn + 16 * (mm >> 2)]) + (mm & 3);
      float sum = 0.f;
      for (int w = 0; w < ks; ++w) sum += src[w * 64 * 4];
      const int m = 16 * t + mm;
      const int64_t col = static_cast<int64_t>(u_begin + pass) * 16 + nn;
      if (m < M && col < N) Y[static_cast<int64_t>(m) * N + col] = sum;
    }
  };

  // x of a chunk, eight rows at a time: each row read contiguously (lane l:
  // values 4 l .. 4 l + 3; rows past M and values past K read as zeros,
  // with no traffic)
  auto x_load = [&](int j, int m0, f32x4m (&v)[8]) {
    const int kc = ((wave * C + j) << 8) + 4 * lane;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int m = m0 + r;
      const int vo = (m < M && kc < K) ? 4 * (m * K + kc) : xrec;
      v[r] = __builtin_bit_cast(f32x4m, __builtin_amdgcn_raw_buffer_load_b128(xrs, vo, 0, 0));
    }
  };
  // ... converted to binary16 and written to the wave's tile in operand
  // order: entry (block b, row m of the 16-row tile, group g) = values
  // 32 b + 4 g .. + 3 (bytes 0-7) and 32 b + 16 + 4 g .. + 3 (bytes 8-15),
  // rows XOR-swizzled by b % 4 so a row's 8-byte writes spread over the
  // banks (lr0: the first of the eight rows within the tile) ...
  auto x_write = [&](int lr0, const f32x4m (&v)[8]) {
    f16x8* tile = xst[wave];
    const int wb = lane >> 3, wg = lane & 3, wh = (lane >> 2) & 1;  // this lane's block, group, half
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int m = lr0 + r;
      const f16x2 h01 = {static_cast<_Float16>(v[r].x), static_cast<_Float16>(v[r].y)};
      const f16x2 h23 = {static_cast<_Float16>(v[r].z), static_cast<_Float16>(v[r].w)};
      uint32_t* e = reinterpret_cast<uint32_t*>(&tile[(wb * 16 + (m ^ (wb & 3))) * 4 + wg]) + 2 * wh;
      e[0] = __builtin_bit_cast(uint32_t, h01);
      e[1] = __builtin_bit_cast(uint32_t, h23);
    }
  };
  // HL: rows 0-3 of x (the rest zero) as hi (tile rows 0-3) and lo (tile
  // rows 4-7) after the chunk's power-of-two scaling of each row; a wide
  // row's operands are zero and its bit is set in xwide[j].  The maxima and
  // minima are wave reductions (one chunk is one wave), so every branch on
  // them is uniform.
  auto x_write_hl = [&](int j, const f32x4m (&v)[8]) {
    f16x8* tile = xst[wave];
    const int wb = lane >> 3, wg = lane & 3, wh = (lane >> 2) & 1;
    uint32_t wm = 0u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4m av = {fabsf(v[r].x), fabsf(v[r].y), fabsf(v[r].z), fabsf(v[r].w)};
      const float a = fmaxf(fmaxf(av.x, av.y), fmaxf(av.z, av.w));
      // smallest nonzero magnitude (+inf when all four are zero; NaN never
      // counts, in neither reduction)
      float z = __builtin_inff();
      z = av.x > 0.f ? fminf(z, av.x) : z;
      z = av.y > 0.f ? fminf(z, av.y) : z;
      z = av.z > 0.f ? fminf(z, av.z) : z;
      z = av.w > 0.f ? fminf(z, av.w) : z;
      const float cmax = wave_max_nonneg(a);
      const float cmin = wave_min_nonneg(z);
      const bool wide = !(cmax < 0x1p124f) || cmin < cmax * 0x1p-20f;
      const int se = scale_exp(__float_as_uint(cmax));
      xu[j][r] = exp2i(-se);
      uint32_t hw0 = 0u, hw1 = 0u, lw0 = 0u, lw1 = 0u;
      if (wide) {
        wm |= 1u << r;
      } else {
        const f32x4m xv = v[r] * exp2i(se);
        const f16x2 h01 = {static_cast<_Float16>(xv.x), static_cast<_Float16>(xv.y)};
        const f16x2 h23 = {static_cast<_Float16>(xv.z), static_cast<_Float16>(xv.w)};
        const f16x2 l01 = {static_cast<_Float16>(xv.x - static_cast<float>(h01[0])),
                           static_cast<_Float16>(xv.y - static_cast<float>(h01[1]))};
        const f16x2 l23 = {static_cast<_Float16>(xv.z - static_cast<float>(h23[0])),
                           static_cast<_Float16>(xv.w - static_cast<float>(h23[1]))};
        hw0 = __builtin_bit_cast(uint32_t, h01);
        hw1 = __builtin_bit_cast(uint32_t, h23);
        lw0 = __builtin_bit_cast(uint32_t, l01);
        lw1 = __builtin_bit_cast(uint32_t, l23);
      }
      uint32_t* eh = reinterpret_cast<uint32_t*>(&tile[(wb * 16 + (r ^ (wb & 3))) * 4 + wg]) + 2 * wh;
      uint32_t* el =
          reinterpret_cast<uint32_t*>(&tile[(wb * 16 + ((4 + r) ^ (wb & 3))) * 4 + wg]) + 2 * wh;
      eh[0] = hw0;
      eh[1] = hw1;
      el[0] = lw0;
      el[1] = lw1;
    }
#pragma unroll
    for (int m = 8; m < 16; ++m) {
      uint32_t* e = reinterpret_cast<uint32_t*>(&tile[(wb * 16 + (m ^ (wb & 3))) * 4 + wg]) + 2 * wh;
      e[0] = 0u;
      e[1] = 0u;
    }
    xwide[j] = wm;
  };
  // ... and lane (m, g) reads its operand of each block.  The tile is the
  // wave's own and LDS operations of a wave complete in order, so no barrier
  // is needed; the empty asm statements with a memory clobber keep the
  // compiler from moving these reads across the tile's writes (which go
  // through another type) on either side.
  auto x_read = [&](int j, int t) {
    const f16x8* tile = xst[wave];
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) xa[j][t][blk] = tile[(blk * 16 + (n ^ (blk & 3))) * 4 + g];
    __asm__ volatile("" ::: "memory");
  };

  if constexpr (C == 1) {
    // two passes in flight, in two register sets; x first and the first two
    // passes' weights right after (the memory counter is in order, so
    // waiting for x never waits for the weights), the later tiles of x
    // eight rows at a time
    uint32_t D0[9], D1[9];
    {
      f32x4m v0[8], v1[8];
      x_load(0, 0, v0);
      if constexpr (!HL) x_load(0, 8, v1);
      load(0, 0, D0);
      load(1, 0, D1);
      if constexpr (HL) {
        x_write_hl(0, v0);
      } else {
        x_write(0, v0);
        x_write(8, v1);
      }
      x_read(0, 0);
#pragma unroll
      for (int t = 1; t < MT; ++t) {
        x_load(0, 16 * t, v0);
        x_write(0, v0);
        x_load(0, 16 * t + 8, v0);
        x_write(8, v0);
        x_read(0, t);
      }
    }
    __syncthreads();  // every wave's operands are in registers: the tiles become partial sums
    int i = 0;
    for (; i + 2 <= npass; i += 2) {
      f32x4m a0[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) a0[t] = f32x4m{0.f, 0.f, 0.f, 0.f};
      compute(0, D0, a0);
      load(i + 2, 0, D0);
      finish(i, a0);
      f32x4m a1[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) a1[t] = f32x4m{0.f, 0.f, 0.f, 0.f};
      compute(0, D1, a1);
      load(i + 3, 0, D1);
      finish(i + 1, a1);
    }
    if (i < npass) {
      f32x4m a0[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) a0[t] = f32x4m{0.f, 0.f, 0.f, 0.f};
      compute(0, D0, a0);
      finish(i, a0);
    }
  } else {
    // one register set per chunk: a chunk's next-pass load is issued as soon
    // as the chunk is computed, so C chunks are in flight during a pass
    uint32_t D[C][9];
    {
      f32x4m v0[8], v1[8];
      x_load(0, 0, v0);
      if constexpr (!HL) x_load(0, 8, v1);
#pragma unroll
      for (int j = 0; j < C; ++j) load(0, j, D[j]);
      if constexpr (HL) {
        x_write_hl(0, v0);
      } else {
        x_write(0, v0);
        x_write(8, v1);
      }
      x_read(0, 0);
      // the later chunks eight rows at a time (registers: the earlier
      // chunks' operands and the weights are live)
#pragma unroll
      for (int j = 1; j < C; ++j) {
        x_load(j, 0, v0);
        if constexpr (HL) {
          x_write_hl(j, v0);
        } else {
          x_write(0, v0);
          x_load(j, 8, v0);
          x_write(8, v0);
        }
        x_read(j, 0);
      }
    }
    __syncthreads();  // every wave's operands are in registers: the tiles become partial sums
    for (int i = 0; i < npass; ++i) {
      f32x4m a[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) a[t] = f32x4m{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < C; ++j) {
        compute(j, D[j], a);
        load(i + 1, j, D[j]);
      }
      finish(i, a);
    }
  }
}

}  // namespace

// Workgroups of the small-M kernel resident on one CU.
int matmul_small_per_cu() {
  // per process (resource use is fixed); racing first calls store the same value
  static std::atomic<int> cache{0};
  int per_cu = cache.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int nb = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, matmul_small_kernel<SM_MAX_M>, SM_THREADS, 0);
    per_cu = (e == hipSuccess && nb > 0) ? nb : 1;
    cache.store(per_cu, std::memory_order_relaxed);
  }
  return per_cu;
}

// The stream16 kernel's shape for (M, K): chunks of 256 K values per wave
// and tiles of 16 rows of x (0: not served).  One tile (M <= 16): up to 16
// chunks one wave each, or up to 24 (K = 6144) in 12 waves of two.  Two or
// three tiles (M <= 48): up to 12 chunks (K = 3072), one per wave (the x
// operands of 48 rows fill 96 registers).  Longer rows stay with the skinny
// kernel: three chunks per wave fit in registers at one tile, but every
// workgroup then reads more x (M x K floats) than the weights of its
// passes; measured slower than the skinny kernel on the 3072 x 9216 down
// projection at 5 to 16 rows (13-14 against 11-12 us).
int matmul_stream16_chunks(int64_t M, int64_t K) {
  if (M < 2 || M > 16 * MS_MAX_MT || K % 64 != 0 || K <= 0) return 0;
  const int64_t nchunk = (K + 255) / 256;
  if (M > 16) return nchunk <= 12 ? 1 : 0;
  if (nchunk <= MS_MAX_WAVES) return 1;
  return nchunk <= 24 ? 2 : 0;
}

template <int C, int MT, bool HL>
static int stream16_per_cu(int threads) {
  // per process and block size (resource use is fixed); racing first calls
  // store the same value
  static std::atomic<int> cache[MS_MAX_WAVES + 1];
  const int w = threads / 64;
  int per_cu = cache[w].load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int nb = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, matmul_stream16_kernel<C, MT, HL>, threads, 0);
    per_cu = (e == hipSuccess && nb > 0) ? nb : 1;
    cache[w].store(per_cu, std::memory_order_relaxed);
  }
  return per_cu;
}

template <int C, int MT, bool HL>
static void launch_stream16(const uint8_t* w, const float* x, float* y, int64_t M, int64_t N,
                            int64_t K, int ks, int cus, hipStream_t s) {
  const int threads = 64 * ks;
  const int64_t units = (N + 15) / 16;
  const int64_t slots = static_cast<int64_t>(stream16_per_cu<C, MT, HL>(threads)) * cus;
  // the fewest passes per workgroup that fit, spread evenly
  const int64_t passes = (units + slots - 1) / slots;
  const unsigned grid = static_cast<unsigned>((units + passes - 1) / passes);
  hipLaunchKernelGGL((matmul_stream16_kernel<C, MT, HL>), dim3(grid), dim3(threads), 0, s, w, x, y,
                     static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
}

hipError_t launch_matmul_stream16(const uint8_t* w, const float* x, float* y, int64_t M,
                                  int64_t N, int64_t K, int cus, hipStream_t s) {
  const int C = matmul_stream16_chunks(M, K);
  if (C == 0) return hipErrorInvalidValue;
  const int ks = static_cast<int>(((K + 255) / 256 + C - 1) / C);
  const int64_t mt = (M + 15) / 16;
  if (M <= 4) {
    if (C == 2)
      launch_stream16<2, 1, true>(w, x, y, M, N, K, ks, cus, s);
    else
      launch_stream16<1, 1, true>(w, x, y, M, N, K, ks, cus, s);
  } else if (C == 2) {
    launch_stream16<2, 1, false>(w, x, y, M, N, K, ks, cus, s);
  } else if (mt == 1) {
    launch_stream16<1, 1, false>(w, x, y, M, N, K, ks, cus, s);
  } else if (mt == 2) {
    launch_stream16<1, 2, false>(w, x, y, M, N, K, ks, cus, s);
  } else {
    launch_stream16<1, 3, false>(w, x, y, M, N, K, ks, cus, s);
  }
  return hipGetLastError();
}

void launch_matmul_small(const uint8_t* w, const float* x, float* y, float* P, int64_t M,
                         int64_t N, int64_t K, int splits, int pps, hipStream_t s) {
  const int tiles = static_cast<int>((N + SM_ROWS - 1) / SM_ROWS);
  hipLaunchKernelGGL(matmul_small_kernel<SM_MAX_M>, dim3(static_cast<unsigned>(tiles * splits)),
                     dim3(SM_THREADS), 0, s, w, x, y, splits > 1 ? P : nullptr,
                     static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), tiles, pps);
}

}  // namespace q4
