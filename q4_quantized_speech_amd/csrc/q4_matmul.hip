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
// Main kernel (K % 64 == 0): a 256-thread workgroup owns a 128 x 128 tile of
// Y; each of its four waves a 64 x 64 sub-tile (4 x 4 MFMA tiles).  K
// advances in stages of 64 (one 36-byte block pair per weight row).  Per
// stage the workgroup converts X and decodes W once into LDS (double
// buffered, in operand order, so fragments are contiguous 1 KiB LDS rows),
// while the global loads of the next three stages are in flight in a ring of
// three register sets (fixed roles in an unrolled loop: no register copies,
// so the in-order vmcnt counter stays exact).  64 KiB of LDS per workgroup
// lets two workgroups share a CU.  Tiles are renumbered so each XCD
// (8 per chip, each with its own L2) works on a contiguous range of tiles that
// share rows of X.
//
// A simple kernel (128 x 128 tiles, one block per stage) covers K % 64 == 32.

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
// Main kernel: 128 x 128 tiles, K % 64 == 0.
// ---------------------------------------------------------------------------
constexpr int T_BM = 128, T_BN = 128, T_THREADS = 256;

// Stage registers of one thread.  Roles are wave-uniform: waves 0-1 stage
// block 0 of the pair, waves 2-3 block 1; thread t stages row t % 128 of X
// and of W for that block.
struct StageRegs {
  f32x4 a[8];     // X: the 32 floats of the block
  uint32_t b[5];  // W: the 20 bytes starting at 16 * block within the pair
};

// Two waves per SIMD is the occupancy target (two workgroups per CU, 64 KiB
// of LDS each); saying so keeps all accumulators in VGPRs.
__global__ __launch_bounds__(T_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void matmul_tile_kernel(const uint8_t* __restrict__ W, const float* __restrict__ X,
                        float* __restrict__ Y, int M, int N, int K, int tiles_n, int ntiles) {
  // [buf][block of the pair][16-row tile][lane]: 2 x 32 KiB
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
  const int lr = tid & 127, blk = tid >> 7;  // row within the tile, block of the pair
  const int am = m0 + lr;
  const float* xrow = X + static_cast<int64_t>(am < M ? am : M - 1) * K + 32 * blk;
  const int bn = n0 + lr;
  const uint8_t* wrow = W + static_cast<int64_t>(bn < N ? bn : N - 1) * rb + 16 * blk;

  auto load = [&](int s, StageRegs& r) {
    s = s < nbp ? s : nbp - 1;  // past the end: reload the last stage (unused)
    const f32x4* xp = reinterpret_cast<const f32x4*>(xrow + 64 * s);
#pragma unroll
    for (int u = 0; u < 8; ++u) r.a[u] = xp[u];
    const uint8_t* wp = wrow + static_cast<int64_t>(s) * PAIR_BYTES;
    const u32x4a p0 = *reinterpret_cast<const u32x4a*>(wp);
    r.b[0] = p0.x; r.b[1] = p0.y; r.b[2] = p0.z; r.b[3] = p0.w;
    r.b[4] = *reinterpret_cast<const uint32_t*>(wp + 16);
  };

  // Ordering guard.  The conversion of a register set is pure arithmetic, so
  // the compiler would hoist it above the barrier to right behind that set's
  // loads, making the wave wait for loads it has just issued.  The first
  // operation on every loaded register is therefore a volatile asm VALU op
  // (the binary16 pack for X, a move for W): volatile asm keeps its place
  // after the barrier, and everything else depends on it.
  auto pk_f16 = [](float a, float b) -> uint32_t {
    uint32_t r;
    asm volatile("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
  };
  auto pin = [](uint32_t v) -> uint32_t {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
  };

  auto store = [&](const StageRegs& r, int buf) {
    // X: lane slot (row % 16) + 16 g holds k {4g..4g+3, 16+4g..16+4g+3}
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 lo = r.a[g], hi = r.a[4 + g];
      const u32x4a h = {pk_f16(lo.x, lo.y), pk_f16(lo.z, lo.w), pk_f16(hi.x, hi.y), pk_f16(hi.z, hi.w)};
      *reinterpret_cast<u32x4a*>(&As[buf][blk][lr >> 4][(lr & 15) + 16 * g]) = h;
    }
    uint32_t b[5];
#pragma unroll
    for (int t = 0; t < 5; ++t) b[t] = pin(r.b[t]);
    if (blk == 0) {  // wave-uniform: bytes 0..19 = scale, codes at byte 2
      const uint32_t d = b[0] & 0xFFFFu;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        Bs[buf][0][lr >> 4][(lr & 15) + 16 * g] = decode8_f16(shift16(b[g + 1], b[g]), d);
    } else {         // bytes 16..35 = (2 bytes of block 0), scale, codes at byte 4
      const uint32_t d = b[0] >> 16;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        Bs[buf][1][lr >> 4][(lr & 15) + 16 * g] = decode8_f16(b[g + 1], d);
    }
  };

  f32x4v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      f16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[buf][bk][wm * 4 + i][lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[buf][bk][wn * 4 + j][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // Three register sets in a ring, two LDS buffers.  Half-step i (stage
  // s + i): issue the loads of stage s + i + 3 into set i % 3 (stored into
  // LDS one half-step earlier), compute from LDS buffer i % 2, then store set
  // (i + 1) % 3 -- stage s + i + 1, loaded two half-steps ago -- into buffer
  // (i + 1) % 2.  Every index is a compile-time constant in the unrolled
  // loop, so no register set is ever copied and the vmcnt waits stay exact.
  StageRegs rs[3];
#define Q4_HALF(I)                                          \
  do {                                                      \
    load(s + (I) + 3, rs[(I) % 3]);                         \
    __builtin_amdgcn_sched_barrier(0);                      \
    compute((I) % 2);                                       \
    store(rs[((I) + 1) % 3], ((I) + 1) % 2);                \
    __syncthreads();                                        \
  } while (0)

  load(0, rs[0]);
  load(1, rs[1]);
  load(2, rs[2]);
  store(rs[0], 0);
  __syncthreads();
  int s = 0;
  for (; s + 6 <= nbp; s += 6) {
    Q4_HALF(0); Q4_HALF(1); Q4_HALF(2); Q4_HALF(3); Q4_HALF(4); Q4_HALF(5);
  }
  // remaining stages (uniform branches; at most five half-steps)
  const int rem = nbp - s;
  if (rem > 0) Q4_HALF(0);
  if (rem > 1) Q4_HALF(1);
  if (rem > 2) Q4_HALF(2);
  if (rem > 3) Q4_HALF(3);
  if (rem > 4) Q4_HALF(4);
#undef Q4_HALF

  // 16 x 16 accumulator layout: lane l holds column l % 16, rows 4 (l / 16) + v.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + v;
      if (row >= M) continue;
      float* yr = Y + static_cast<int64_t>(row) * N;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + (lane & 15);
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
