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
  // into hi/lo binary16 and stored in operand order.
  auto stage_store = [&](const f32x4m (&v)[MR]) {
    const int k = 4 * lane, blk = wave * 8 + (k >> 5), e = k & 31;
    const int gg = (e & 15) >> 2, half = e >> 4;  // operand group, low/high nibble half
#pragma unroll
    for (int u = 0; u < MR; ++u) {
      if (u < M) {
        const float a = fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w)));
        const int se = scale_exp(__float_as_uint(wave_max_nonneg(a)));
        const f32x4m xv = v[u] * exp2i(se);
        const f16x2 h01 = {static_cast<_Float16>(xv.x), static_cast<_Float16>(xv.y)};
        const f16x2 h23 = {static_cast<_Float16>(xv.z), static_cast<_Float16>(xv.w)};
        const f16x2 l01 = {static_cast<_Float16>(xv.x - static_cast<float>(h01[0])),
                           static_cast<_Float16>(xv.y - static_cast<float>(h01[1]))};
        const f16x2 l23 = {static_cast<_Float16>(xv.z - static_cast<float>(h23[0])),
                           static_cast<_Float16>(xv.w - static_cast<float>(h23[1]))};
        uint32_t* ph = reinterpret_cast<uint32_t*>(&xh[blk][gg][u]) + 2 * half;
        uint32_t* pl = reinterpret_cast<uint32_t*>(&xl[blk][gg][u]) + 2 * half;
        ph[0] = __builtin_bit_cast(uint32_t, h01);
        ph[1] = __builtin_bit_cast(uint32_t, h23);
        pl[0] = __builtin_bit_cast(uint32_t, l01);
        pl[1] = __builtin_bit_cast(uint32_t, l23);
        if (lane == 0) usc[wave][u >> 2][u & 3] = exp2i(-se);
      }
    }
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

}  // namespace

// Workgroups of the small-M kernel resident on one CU.
int matmul_small_per_cu() {
  static int per_cu = 0;  // per process; resource use is fixed
  if (per_cu == 0) {
    int nb = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, matmul_small_kernel<SM_MAX_M>, SM_THREADS, 0);
    per_cu = (e == hipSuccess && nb > 0) ? nb : 1;
  }
  return per_cu;
}

void launch_matmul_small(const uint8_t* w, const float* x, float* y, float* P, int64_t M,
                         int64_t N, int64_t K, int splits, int pps, hipStream_t s) {
  const int tiles = static_cast<int>((N + SM_ROWS - 1) / SM_ROWS);
  hipLaunchKernelGGL(matmul_small_kernel<SM_MAX_M>, dim3(static_cast<unsigned>(tiles * splits)),
                     dim3(SM_THREADS), 0, s, w, x, y, splits > 1 ? P : nullptr,
                     static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), tiles, pps);
}

}  // namespace q4
