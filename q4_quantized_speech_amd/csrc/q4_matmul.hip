// Q4_0 matrix-matrix product on the CDNA4 matrix cores: Y = X * deq(W)^T.
//
// Section "Architecture" of "Implémentation en Rust du modèle Voxtral Mini 4B
// Realtime de Mistral pour l'exécuter dans le navigateur": the audio encoder
// (width 1280) and the adapter after the 4x convolutional downsample run their
// projections over many frames at once, and the decoder's prompt prefix (38,
// 76 tokens: section "Correction du padding Q4") does the same for several
// tokens; these are dense contractions, so they go to v_mfma_f32_16x16x32_f16.
//
// Operand order.  The MFMA sums over k, so any permutation of k applied to
// both operands gives the same products.  Lane l = i + 16 g (i < 16, g < 4)
// carries row/column i and the eight k values {4g..4g+3, 16+4g..16+4g+3} of a
// Q4_0 block: exactly the low and high nibbles of the four code bytes
// qs[4g..4g+3], so one dword of codes is one lane's operand.  Decoding is
// (q - 8) * d in binary16 (exact q - 8, one rounding of the product); X is
// rounded to binary16 (nearest even); accumulation is float32.
//
// Main kernel (K % 64 == 0): a 256-thread workgroup owns a 128 (M) x 256 (N)
// tile of Y; each of its four waves a 64 x 128 sub-tile (4 x 8 MFMA tiles).
// K advances in stages of 64 (one 36-byte block pair per weight row).  Per
// stage the workgroup converts X and decodes W once into LDS (double
// buffered, in operand order, so fragments are contiguous 1 KiB LDS rows),
// while the global loads of the stage after next are already in flight in a
// second register set (two sets used alternately: no register copies, so the
// in-order vmcnt counter stays exact).  Tiles are renumbered so each XCD
// (8 per chip, each with its own L2) works on a contiguous range of tiles that
// share rows of X.
//
// A simple kernel (128 x 128 tiles, one block per stage) covers any K % 32.

#include "q4_device.h"
#include "q4_kernels.h"

namespace q4 {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));

// Decode the 8 codes of one qs dword into binary16 (q - 8) * d, operand order.
__device__ __forceinline__ f16x8 decode8_f16(uint32_t qs, uint32_t d16) {
  const uint32_t lo = qs & 0x0F0F0F0Fu;
  const uint32_t hi = (qs >> 4) & 0x0F0F0F0Fu;
  // v_perm places a code in the low byte of each half with 0x64 above it:
  // the binary16 value 1024 + q; subtracting 1032 leaves q - 8 exactly.
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

// Tile renumbering: the hardware deals workgroups to the 8 XCDs round-robin;
// give XCD x the tiles [x*G/8, (x+1)*G/8) so neighbouring tiles share an L2.
__device__ __forceinline__ int xcd_tile(int bid, int ntiles) {
  constexpr int XCD = 8;
  const int per = ntiles / XCD, rem = ntiles % XCD;
  const int x = bid % XCD, i = bid / XCD;
  // the first `rem` XCDs take one extra tile
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + i;
}

// ---------------------------------------------------------------------------
// Main kernel: 128 x 256 tiles, K % 64 == 0.
// ---------------------------------------------------------------------------
constexpr int T_BM = 128, T_BN = 256, T_THREADS = 256;

struct StageRegs {
  f32x4 a[8];     // X: row tid/2, 32 floats of block (tid & 1)
  uint32_t b[9];  // W: row tid, one 36-byte block pair
};

__global__ __launch_bounds__(T_THREADS) void matmul_tile_kernel(
    const uint8_t* __restrict__ W, const float* __restrict__ X, float* __restrict__ Y, int M, int N,
    int K, int tiles_n, int ntiles) {
  // [buf][block of the pair][16-row tile][lane]
  __shared__ f16x8 As[2][2][T_BM / 16][64];
  __shared__ f16x8 Bs[2][2][T_BN / 16][64];

  const int tile = xcd_tile(blockIdx.x, ntiles);
  const int m0 = (tile / tiles_n) * T_BM;
  const int n0 = (tile % tiles_n) * T_BN;
  const int nbp = K >> 6;  // stages
  const int64_t rb = static_cast<int64_t>(nbp) * PAIR_BYTES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // loader roles.  Rows past M and columns past N are clamped to the last
  // valid one: they only feed outputs that are never stored, so no masking
  // (a mask on loaded data would pull a wait for this stage's loads forward).
  const int ar = tid >> 1, ah = tid & 1;  // X row within the tile, block of the pair
  const int am = m0 + ar;
  const float* xrow = X + static_cast<int64_t>(am < M ? am : M - 1) * K + 32 * ah;
  const int bn = n0 + tid;
  const uint8_t* wrow = W + static_cast<int64_t>(bn < N ? bn : N - 1) * rb;

  auto load = [&](int s, StageRegs& r) {
    s = s < nbp ? s : nbp - 1;  // past the end: reload the last stage (unused)
    const f32x4* xp = reinterpret_cast<const f32x4*>(xrow + 64 * s);
#pragma unroll
    for (int u = 0; u < 8; ++u) r.a[u] = xp[u];
    const uint8_t* wp = wrow + static_cast<int64_t>(s) * PAIR_BYTES;
    const u32x4a p0 = *reinterpret_cast<const u32x4a*>(wp);
    const u32x4a p1 = *reinterpret_cast<const u32x4a*>(wp + 16);
    r.b[0] = p0.x; r.b[1] = p0.y; r.b[2] = p0.z; r.b[3] = p0.w;
    r.b[4] = p1.x; r.b[5] = p1.y; r.b[6] = p1.z; r.b[7] = p1.w;
    r.b[8] = *reinterpret_cast<const uint32_t*>(wp + 32);
  };
  auto store = [&](const StageRegs& r, int buf, uint32_t z) {
    auto zf = [z](f32x4 v) {
      return f32x4{__uint_as_float(__float_as_uint(v.x) | z), __uint_as_float(__float_as_uint(v.y) | z),
                   __uint_as_float(__float_as_uint(v.z) | z), __uint_as_float(__float_as_uint(v.w) | z)};
    };
    // X: lane slot (row % 16) + 16 g holds k {4g..4g+3, 16+4g..16+4g+3}
#pragma unroll
    for (int g = 0; g < 4; ++g)
      As[buf][ah][ar >> 4][(ar & 15) + 16 * g] = cvt8_f16(zf(r.a[g]), zf(r.a[4 + g]));
    // W: block 0 (scale in the low half of dword 0, codes shifted by 2 bytes),
    //    block 1 (scale in the high half of dword 4, codes in dwords 5..8)
    uint32_t b[9];
#pragma unroll
    for (int t = 0; t < 9; ++t) b[t] = r.b[t] | z;
    const uint32_t d0 = b[0] & 0xFFFFu;
    const uint32_t d1 = b[4] >> 16;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      Bs[buf][0][tid >> 4][(tid & 15) + 16 * g] = decode8_f16(shift16(b[g + 1], b[g]), d0);
      Bs[buf][1][tid >> 4][(tid & 15) + 16 * g] = decode8_f16(b[5 + g], d1);
    }
  };

  f32x4v acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      f16x8 a[4], b[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[buf][blk][wm * 4 + i][lane];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = Bs[buf][blk][wn * 8 + j][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // Ordering guard.  The conversion of a register set is pure arithmetic, so
  // the compiler may hoist it above the barrier to right behind that set's
  // loads, making the wave wait for loads it has just issued.  The conversion
  // ORs its inputs with a zero read from LDS after the barrier, which ties it
  // below that point without reading the set any earlier.
  // The word is read inline through the LDS variable, not volatile and not
  // through a lambda capture: either would make it a flat load, which counts
  // on vmcnt and would wait for the global loads.  The stored value is a
  // runtime zero (K > 0) so the compiler cannot fold the reads, and a read
  // after a barrier cannot move above it.
  __shared__ uint32_t zero_word;
  if (tid == 0) zero_word = static_cast<uint32_t>(K) >> 31;

  StageRegs r0, r1;
  load(0, r0);
  load(1, r1);
  __syncthreads();  // zero_word is visible
  store(r0, 0, 0u);
  __syncthreads();
  uint32_t z = zero_word;
  // Entering with s even: LDS buf 0 holds stage s, r1 holds stage s+1.  Each
  // half-step issues the loads two stages ahead, computes one stage and
  // stores the next; one exit keeps the accumulators in place.
  int s = 0;
  for (; s + 1 < nbp; s += 2) {
    load(s + 2, r0);
    __builtin_amdgcn_sched_barrier(0);  // issue the loads before the compute
    compute(0);
    store(r1, 1, z);
    __syncthreads();
    z = zero_word;
    load(s + 3, r1);
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    store(r0, 0, z);
    __syncthreads();
    z = zero_word;
  }
  if (s < nbp) compute(0);  // odd number of stages: the last one is in buf 0

  // 16 x 16 accumulator layout: lane l holds column l % 16, rows 4 (l / 16) + v.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + v;
      if (row >= M) continue;
      float* yr = Y + static_cast<int64_t>(row) * N;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = n0 + wn * 128 + j * 16 + (lane & 15);
        if (col < N) yr[col] = acc[i][j][v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Simple kernel: 128 x 128 tiles, one block per stage, any K % 32 == 0.
// ---------------------------------------------------------------------------
constexpr int S_BM = 128, S_BN = 128, S_THREADS = 256;

__global__ __launch_bounds__(S_THREADS) void matmul_simple_kernel(
    const uint8_t* __restrict__ W, const float* __restrict__ X, float* __restrict__ Y, int M, int N,
    int K) {
  __shared__ f16x8 As[2][S_BM / 16][64];
  __shared__ f16x8 Bs[2][S_BN / 16][64];

  const int nb = K / QK;
  const int m0 = blockIdx.y * S_BM;
  const int n0 = blockIdx.x * S_BN;
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
      const int it = tid + S_THREADS * u;
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
      const int it = tid + S_THREADS * u;
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
  if (K % 64 == 0) {
    const int tiles_n = static_cast<int>((N + T_BN - 1) / T_BN);
    const int tiles_m = static_cast<int>((M + T_BM - 1) / T_BM);
    const int ntiles = tiles_n * tiles_m;
    hipLaunchKernelGGL(matmul_tile_kernel, dim3(ntiles), dim3(T_THREADS), 0, s, w, x, y,
                       static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), tiles_n,
                       ntiles);
  } else {
    const dim3 grid(static_cast<unsigned>((N + S_BN - 1) / S_BN),
                    static_cast<unsigned>((M + S_BM - 1) / S_BM));
    hipLaunchKernelGGL(matmul_simple_kernel, grid, dim3(S_THREADS), 0, s, w, x, y,
                       static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
  }
  return hipGetLastError();
}

}  // namespace q4
