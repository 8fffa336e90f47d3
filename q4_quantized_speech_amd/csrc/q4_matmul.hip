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
// Kernels, by shape (the planner at the end of this file picks one): the
// wave-specialised kernel for outputs at least 512 wide (the encoder and the
// adapter, and prompt prefixes past 48 rows: BM x 256 tiles, loading waves
// decode, multiplying waves only read LDS), the skinny kernel for the
// prompt-prefix shapes up to 48 rows that the stream16 kernel does not take
// (W streams through the MFMA A operand), the tile kernel below for narrower
// outputs, the simple kernel for K % 64 == 32; up to 4 rows of X go to the
// matvec or to the small-M kernel, 3 to 48 rows mostly to the stream16
// kernel (q4_smallm.hip).
//
// Tile kernel (K % 64 == 0): a 256-thread workgroup owns a 128 x 128 tile of
// Y; each of its four waves a 64 x 64 sub-tile (4 x 4 MFMA tiles).  K
// advances in stages of 64 (one 36-byte block pair per weight row).  Global
// loads are coalesced (16 lanes read one row of X; consecutive lanes read
// consecutive dwords of the stage's weight bytes) and go through range-checked
// buffer resources, so rows past M or N read as zeros.  Per stage the
// workgroup converts X to binary16 and decodes W (from raw codes staged in LDS
// one stage earlier) into LDS in operand order, double buffered, while the
// loads of later stages are in flight in a ring of three register sets.  73
// KiB of LDS per workgroup lets two workgroups share a CU.  When the tiles
// cannot fill the GPU (any of the kernels), K is split over several
// workgroups per tile; their partial tiles go to a workspace and a second
// kernel adds them in a fixed order.  Tiles are renumbered so each XCD (8 per chip, each with its own L2)
// works on a contiguous range of tiles that share rows of X.
//
// A simple kernel (128 x 128 tiles, one block per stage) covers K % 64 == 32.

#include <algorithm>
#include <cstdint>

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
// Main kernel: 128 x BN tiles (BN = 128 or 256), K % 64 == 0, K optionally
// split over several workgroups per tile.
// ---------------------------------------------------------------------------
constexpr int T_BM = 128;
constexpr int MAX_SPLITS = 16;

// Cache policy of the GEMMs' output stores (Y, or the K split's partial
// slices): sc0 sc1, written through to memory as they are produced rather
// than left dirty in the L2 for the end of the kernel.  Measured on the
// wide kernel (same box, alternating builds): encoder layer + adapter at
// M = 1500 125.8-129.3 -> 121.9 us, at M = 375 78.7 -> 76.2, at M = 3000
// 226.7 -> 221.7; on Y alone it gained little (125.0 at M = 1500), so most
// of it is the partial slices that the fold kernel reads next.
constexpr int WRITE_THROUGH = 17;  // the sc0 and sc1 bits of the buffer instruction

// Raw buffer resource over [base, base + bytes): 32-bit data, range checked,
// so loads past the end return zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : static_cast<int>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

template <int BN>
struct TileCfg {
  static constexpr int THREADS = 2 * BN;            // 8 or 4 waves: 2 along M, BN / 64 along N
  static constexpr int WN = BN / 64;
  static constexpr int XRS = THREADS / 16;          // rows per X load round
  static constexpr int XU = T_BM / XRS;             // X load rounds (16-byte chunks per thread)
  static constexpr int WROWS = THREADS / 9;         // rows per W load round
  static constexpr int WLANES = 9 * WROWS;
  static constexpr int WFULL = BN / WROWS;          // full W rounds
  static constexpr int WLAST = BN - WFULL * WROWS;  // rows of the last round
  static constexpr int WU = WFULL + (WLAST > 0);
  static constexpr int WRAW = 9 * BN;               // code dwords of one stage
  static_assert(WFULL * WLANES + 9 * WLAST == WRAW, "code loads cover the stage");
  static_assert(XU * XRS == T_BM, "X loads cover the tile");
};

template <int BN, int D>
struct StageRing {
  f32x4 x[D][TileCfg<BN>::XU];
  uint32_t w[D][TileCfg<BN>::WU];
};

// Loader roles (thread t).
//  X: j = t % 16 is a 16-byte chunk of a row's 256-byte stage span, r = t / 16
//     a row; rows r + XRS u.  Sixteen lanes read one row's span, so one load
//     instruction covers four whole rows (a lane per row would touch 64 cache
//     lines per instruction and saturate the address unit).  Chunk j holds
//     k = 4 j .. 4 j + 3: block j / 8, slot g = j % 4, low half (k 4g..4g+3)
//     if j % 8 < 4, else high half (k 16+4g..16+4g+3).
//  W: the stage's BN rows x 36 bytes, loaded in rounds of WROWS rows x 9
//     dwords: consecutive lanes read consecutive dwords of a row.  They go to
//     LDS as they are (9 dwords a row) and are decoded one stage later by
//     thread (row t % BN, block t / BN).
// LDS: X in operand order, swizzled so that both the 8-byte writes of a row's
// 16 lanes and the 16-byte operand reads hit distinct banks: slot g of row
// r (block b) sits at element 16 g + (r % 16 ^ (g + 4 b)) of its 16-row tile.
// One resource per load round makes rows past M or N read as zeros.
//
// Pipeline over the stages t of this split (buffers and register sets indexed
// by t, compile-time constants in the unrolled loop).  Step t: issue the loads
// of X(t + D) and W(t + D + 1); multiply stage t from LDS buffer t % 2; decode
// the raw codes of stage t + 1 into buffer (t + 1) % 2; convert X(t + 1) into
// buffer (t + 1) % 2; put the raw codes of stage t + 2 into raw buffer t % 2;
// barrier.  Loads have D - 1 steps to arrive.
template <int BN, int D>
__global__ __launch_bounds__(TileCfg<BN>::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void matmul_tile_kernel(const uint8_t* __restrict__ W, const float* __restrict__ X,
                        float* __restrict__ Y, float* __restrict__ P, int M, int N, int K,
                        int tiles_n, int ntiles, int split_stages) {
  using C = TileCfg<BN>;
  __shared__ f16x8 As[2][2][T_BM / 16][64];  // [buf][block][16-row tile][element]
  __shared__ f16x8 Bs[2][2][BN / 16][64];
  __shared__ uint32_t Wraw[2][C::WRAW];

  const int item = xcd_tile(blockIdx.x, gridDim.x);
  const int split = item / ntiles, tile = item % ntiles;
  const int m0 = (tile / tiles_n) * T_BM;
  const int n0 = (tile % tiles_n) * BN;
  const int nbp = K >> 6;
  const int s0 = split * split_stages;
  const int nst = min(nbp - s0, split_stages);  // >= 1 (host guarantees)
  const int64_t rb = static_cast<int64_t>(nbp) * PAIR_BYTES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;

  const int xj = tid & 15, xr = tid >> 4;
  __amdgpu_buffer_rsrc_t xrs[C::XU];
#pragma unroll
  for (int u = 0; u < C::XU; ++u)
    xrs[u] = make_rsrc(X + static_cast<int64_t>(m0 + C::XRS * u) * K,
                       static_cast<int64_t>(M - m0 - C::XRS * u) * K * 4);
  const int xvo = xr * K * 4 + xj * 16;
  const int xb = xj >> 3, xh = (xj >> 2) & 1, xg = xj & 3;
  const int xe = 16 * xg + ((xr & 15) ^ (xg + 4 * xb));

  __amdgpu_buffer_rsrc_t wrs[C::WU];
#pragma unroll
  for (int u = 0; u < C::WU; ++u)
    wrs[u] = make_rsrc(W + static_cast<int64_t>(n0 + C::WROWS * u) * rb,
                       static_cast<int64_t>(N - n0 - C::WROWS * u) * rb);
  const int wq = tid / 9;
  const int wvo = static_cast<int>(wq * rb) + (tid - 9 * wq) * 4;
  const bool wlane = tid < C::WLANES, wlast = tid < 9 * C::WLAST;
  const int lr = tid % BN, blk = tid / BN;  // decode role: row, block of the pair

  StageRing<BN, D> ring;
  auto load_x = [&](int t, int slot) {
    const int so = (s0 + (t < nst ? t : nst - 1)) * 256;
#pragma unroll
    for (int u = 0; u < C::XU; ++u)
      ring.x[slot][u] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs[u], xvo, so, 0));
  };
  auto load_w = [&](int t, int slot) {
    const int so = (s0 + (t < nst ? t : nst - 1)) * PAIR_BYTES;
    if (wlane) {
#pragma unroll
      for (int u = 0; u < C::WFULL; ++u)
        ring.w[slot][u] = __builtin_amdgcn_raw_buffer_load_b32(wrs[u], wvo, so, 0);
    }
    if constexpr (C::WLAST > 0) {
      if (wlast) ring.w[slot][C::WFULL] = __builtin_amdgcn_raw_buffer_load_b32(wrs[C::WFULL], wvo, so, 0);
    }
  };

  // Ordering guard.  Conversions of loaded registers are pure arithmetic, so
  // the compiler would hoist them to right behind their loads, making the
  // wave wait for loads it has just issued.  The first operation on every
  // loaded register is a volatile asm op (the binary16 pack for X, a move for
  // W), which keeps its place in the program; everything else depends on it.
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

  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  auto store_x = [&](int slot, int buf) {
    char* base = reinterpret_cast<char*>(&As[buf][xb][xr >> 4][xe]) + 8 * xh;
#pragma unroll
    for (int u = 0; u < C::XU; ++u) {
      const f32x4 v = ring.x[slot][u];
      const u32x2 h = {pk_f16(v.x, v.y), pk_f16(v.z, v.w)};
      *reinterpret_cast<u32x2*>(base + u * (C::XRS / 16) * 64 * 16) = h;
    }
  };
  auto store_w = [&](int slot, int buf) {
    if (wlane) {
#pragma unroll
      for (int u = 0; u < C::WFULL; ++u) Wraw[buf][C::WLANES * u + tid] = pin(ring.w[slot][u]);
    }
    if constexpr (C::WLAST > 0) {
      if (wlast) Wraw[buf][C::WLANES * C::WFULL + tid] = pin(ring.w[slot][C::WFULL]);
    }
  };
  auto decode = [&](int buf) {
    const uint32_t* wr = &Wraw[buf][lr * 9 + blk * 4];
    uint32_t b[5];
#pragma unroll
    for (int t = 0; t < 5; ++t) b[t] = wr[t];
    if (blk == 0) {  // wave-uniform: bytes 0..19 = scale, codes from byte 2
      const uint32_t d = b[0] & 0xFFFFu;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        Bs[buf][0][lr >> 4][(lr & 15) + 16 * g] = decode8_f16(shift16(b[g + 1], b[g]), d);
    } else {         // bytes 16..35 = 2 bytes of block 0, scale, codes from byte 20
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

  // operand element of this lane in each block (swizzled X, plain W)
  const int ag = lane >> 4;
  const int ae0 = 16 * ag + ((lane & 15) ^ ag);
  const int ae1 = 16 * ag + ((lane & 15) ^ (ag + 4));
  auto compute = [&](int buf) {
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      f16x8 a[4], b[4];
      const int ae = bk ? ae1 : ae0;
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[buf][bk][wm * 4 + i][ae];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[buf][bk][wn * 4 + j][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

#define Q4_STEP(I)                                          \
  do {                                                      \
    load_x(t + (I) + D, (I) % D);                           \
    load_w(t + (I) + D + 1, (I) % D);                       \
    __builtin_amdgcn_sched_barrier(0);                      \
    compute((I) % 2);                                       \
    decode(((I) + 1) % 2);                                  \
    store_x(((I) + 1) % D, ((I) + 1) % 2);                  \
    store_w(((I) + 1) % D, (I) % 2);                        \
    __syncthreads();                                        \
  } while (0)

  // prologue: stage 0 converted, raw codes of stages 0 and 1 in LDS, stage 0
  // decoded; X(1 .. D-1) and W(2 .. D) in flight in ring slots 1 .. D-1.
  load_x(0, 0);
  load_w(0, 0);
  load_w(1, 1);
  store_w(0, 0);
  store_w(1, 1);
  store_x(0, 0);
#pragma unroll
  for (int i = 1; i < D; ++i) {
    load_x(i, i);
    load_w(i + 1, i);
  }
  __syncthreads();
  decode(0);
  __syncthreads();
  int t = 0;
  if constexpr (D == 3) {
    for (; t + 6 <= nst; t += 6) {
      Q4_STEP(0); Q4_STEP(1); Q4_STEP(2); Q4_STEP(3); Q4_STEP(4); Q4_STEP(5);
    }
    const int rem = nst - t;  // uniform; at most five more steps
    if (rem > 0) Q4_STEP(0);
    if (rem > 1) Q4_STEP(1);
    if (rem > 2) Q4_STEP(2);
    if (rem > 3) Q4_STEP(3);
    if (rem > 4) Q4_STEP(4);
  } else {
    static_assert(D == 4, "prefetch depth 3 or 4");
    for (; t + 4 <= nst; t += 4) {
      Q4_STEP(0); Q4_STEP(1); Q4_STEP(2); Q4_STEP(3);
    }
    const int rem = nst - t;  // uniform; at most three more steps
    if (rem > 0) Q4_STEP(0);
    if (rem > 1) Q4_STEP(1);
    if (rem > 2) Q4_STEP(2);
  }
#undef Q4_STEP

  // 16 x 16 accumulator layout: lane l holds column l % 16, rows 4 (l / 16) + v.
  // With a split, partial sums go to slice `split` of P ([splits][M][N]).
  float* out = P ? P + static_cast<int64_t>(split) * M * N : Y;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + v;
      if (row >= M) continue;
      float* yr = out + static_cast<int64_t>(row) * N;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + (lane & 15);
        if (col < N) yr[col] = acc[i][j][v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wave-specialised kernel: BM x 256 tiles (BM = 128, 96, 64 or 32; the
// shorter tiles fill the GPU where M gives few tiles), 512 threads, K % 64 == 0.
// Waves 0-3 multiply, each a BM x 64 slice (BM/16 x 4 MFMA tiles).  Waves 4-7 load a stage D stages ahead (each thread one weight
// row's 36-byte block pair and 16-byte chunks of X), convert X to binary16
// and decode the row's first block into binary16 (q - 8) d in operand order;
// the second block's codes and scale go to LDS raw (4 dwords per row: the
// 64 lanes of a fragment read hit 64 distinct banks) and the multiplying
// waves decode them right before use.  Each weight is decoded once.  One
// barrier per stage.  Measured on the encoder shapes: splitting the decode
// this way ran 1-4 % faster than either side decoding both blocks, and D = 2
// faster than deeper rings.
// ---------------------------------------------------------------------------
constexpr int WS_BN = 256, WS_D = 2;
constexpr int WS_CONS = 256, WS_PT = 256, WS_THREADS = WS_CONS + WS_PT;
constexpr int WS_WU = 9;                       // code dwords per producer thread: one pair
static_assert(WS_PT == WS_BN, "one weight row per producer thread");

// RES (no K split): Y = R + the product, the add in float32 after the
// accumulation, R read at the offsets Y is written (R may be Y itself).  The
// kernels below wrap this body: the plain one keeps Y restrict-qualified
// (without it the compiler scheduled the main loop differently, 1-2 %
// slower), the residual one cannot (R may be Y).
template <int BM, bool RES>
__device__ __forceinline__ void ws_body(const uint8_t* __restrict__ W, const float* __restrict__ X,
                                        float* Y, float* P, const float* R, int M, int N, int K,
                                        int tiles_n, int ntiles, int split_stages) {
  constexpr int MI = BM / 16;                 // 16-row tiles of X
  constexpr int XU = BM * 16 / WS_PT;         // 16-byte X chunks per producer thread
  static_assert(BM % 32 == 0 && BM >= 32 && BM <= 128, "X is loaded in rounds of 32 rows");
  __shared__ f16x8 As[2][2][MI][64];          // [buf][block][16-row tile][element]
  __shared__ f16x8 Bs[2][WS_BN / 16][64];     // [buf][16-row fragment][lane]: block 0, binary16
  __shared__ __attribute__((aligned(16))) uint32_t Wc[2][WS_BN * 4];  // block 1 raw codes, 4 dwords per row
  __shared__ uint16_t Wsc[2][WS_BN];          // block 1 scales

  const int item = xcd_tile(blockIdx.x, gridDim.x);
  const int split = item / ntiles, tile = item % ntiles;
  const int m0 = (tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * WS_BN;
  const int nbp = K >> 6;
  const int s0 = split * split_stages;
  const int nst = min(nbp - s0, split_stages);  // >= 1 (host guarantees)
  const int64_t rb = static_cast<int64_t>(nbp) * PAIR_BYTES;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;  // wave-uniform role

  if (wave < 4) {
    // ------------------------------ multiply ------------------------------
    const int lane = tid & 63;
    const int ag = lane >> 4;
    const int ae0 = 16 * ag + ((lane & 15) ^ ag);
    const int ae1 = 16 * ag + ((lane & 15) ^ (ag + 4));
    f32x4v acc[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int buf) {
#pragma unroll
      for (int bk = 0; bk < 2; ++bk) {
        f16x8 b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // first block: decoded by the loading waves; second block: code
          // dword ag of this lane's weight row, decoded here
          if (bk == 0) {
            b[j] = Bs[buf][4 * wave + j][lane];
          } else {
            const int row = 64 * wave + 16 * j + (lane & 15);
            b[j] = decode8_f16(Wc[buf][row * 4 + ag], Wsc[buf][row]);
          }
        }
        const int ae = bk ? ae1 : ae0;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const f16x8 a = As[buf][bk][i][ae];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[j], acc[i][j], 0, 0, 0);
        }
      }
    };
    __syncthreads();  // prologue: stage 0 in LDS
    int t = 0;
    for (; t + 2 <= nst; t += 2) {
      compute(0);
      __syncthreads();
      compute(1);
      __syncthreads();
    }
    if (t < nst) {
      compute(0);
      __syncthreads();
    }
    float* out = P ? P + static_cast<int64_t>(split) * M * N : Y;
    if (n0 + WS_BN <= N && N < (1 << 22)) {
      // whole columns: range-checked stores drop the rows past M, no branches
      // (32-bit offsets: 128 rows of N floats stay below 2^31 bytes)
      const int rows = min(M - m0, BM);
      const __amdgpu_buffer_rsrc_t yrs =
          make_rsrc(out + static_cast<int64_t>(m0) * N, static_cast<int64_t>(rows) * N * 4);
      const int cb = (n0 + wave * 64 + (lane & 15)) * 4;
      if constexpr (RES) {
        // the residual tile in groups of 4 row tiles (64 values per lane),
        // each group's loads in flight together before its adds and stores
        const __amdgpu_buffer_rsrc_t rrs =
            make_rsrc(R + static_cast<int64_t>(m0) * N, static_cast<int64_t>(rows) * N * 4);
        constexpr int GI = MI < 4 ? MI : 4;
#pragma unroll
        for (int i0 = 0; i0 < MI; i0 += GI) {
          float rv[GI][4][4];
#pragma unroll
          for (int ii = 0; ii < GI; ++ii)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int ro = ((i0 + ii) * 16 + (lane >> 4) * 4 + v) * N * 4 + cb;
#pragma unroll
              for (int j = 0; j < 4; ++j)
                rv[ii][v][j] = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(rrs, ro + j * 64, 0, 0));
            }
#pragma unroll
          for (int ii = 0; ii < GI; ++ii)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int ro = ((i0 + ii) * 16 + (lane >> 4) * 4 + v) * N * 4 + cb;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float val = acc[i0 + ii][j][v] + rv[ii][v][j];
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), yrs, ro + j * 64, 0,
                                                      WRITE_THROUGH);
              }
            }
        }
      } else {
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int ro = (i * 16 + (lane >> 4) * 4 + v) * N * 4 + cb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float val = acc[i][j][v];
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), yrs, ro + j * 64, 0,
                                                    WRITE_THROUGH);
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = m0 + i * 16 + (lane >> 4) * 4 + v;
          if (row >= M) continue;
          float* yr = out + static_cast<int64_t>(row) * N;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = n0 + wave * 64 + j * 16 + (lane & 15);
            if (col < N) {
              if constexpr (RES)
                yr[col] = acc[i][j][v] + R[static_cast<int64_t>(row) * N + col];
              else
                yr[col] = acc[i][j][v];
            }
          }
        }
      }
    }
  } else {
    // ------------------------------- prepare -------------------------------
    const int tp = tid - WS_CONS;  // 0 .. 255
    // On tiles of up to 96 rows the loading waves' stage (loads, convert,
    // decode, LDS writes) is as long as the multiplying waves' MFMAs: issue
    // ahead of them on the shared SIMDs (measured, same box: M = 375 encoder
    // layer 83.5 -> 81.5 us; on 128-row tiles it cost ~1 %, so not there).
    if constexpr (BM <= 96) __builtin_amdgcn_s_setprio(3);
    // X: one A-operand entry per round -- elements 4g..4g+3 and 16+4g..+3 of
    // block xb of row xr + 32 u (two 16-byte loads, one 16-byte LDS write;
    // the 8 lanes of a write cycle hit 8 distinct bank groups)
    const int xg = tp & 3, xb = (tp >> 2) & 1, xr = tp >> 3;
    __amdgpu_buffer_rsrc_t xrs[XU / 2];
#pragma unroll
    for (int u = 0; u < XU / 2; ++u)
      xrs[u] = make_rsrc(X + static_cast<int64_t>(m0 + 32 * u) * K,
                         static_cast<int64_t>(M - m0 - 32 * u) * K * 4);
    const int xvo = xr * K * 4 + xb * 128 + xg * 16;
    const int xe = 16 * xg + ((xr & 15) ^ (xg + 4 * xb));
    // W: this thread's weight row n0 + tp, one 36-byte pair per stage
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(W + static_cast<int64_t>(n0) * rb,
                                                 static_cast<int64_t>(N - n0) * rb);
    const int wvo = static_cast<int>(tp * rb);

    f32x4 rx[WS_D][XU];
    uint32_t rw[WS_D][WS_WU];
    auto load = [&](int t, int slot) {
      const int st = s0 + (t < nst ? t : nst - 1);
#pragma unroll
      for (int u = 0; u < XU / 2; ++u) {
        rx[slot][2 * u] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs[u], xvo, st * 256, 0));
        rx[slot][2 * u + 1] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs[u], xvo + 64, st * 256, 0));
      }
      const int wo = wvo + st * PAIR_BYTES;
      const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wo, 0, 0));
      const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wo, 16, 0));
      rw[slot][0] = a.x; rw[slot][1] = a.y; rw[slot][2] = a.z; rw[slot][3] = a.w;
      rw[slot][4] = b.x; rw[slot][5] = b.y; rw[slot][6] = b.z; rw[slot][7] = b.w;
      rw[slot][8] = __builtin_amdgcn_raw_buffer_load_b32(wrs, wo, 32, 0);
    };
    auto pk_f16 = [](float a, float b) -> uint32_t {
      uint32_t r;
      asm volatile("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
      return r;
    };
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    auto store = [&](int slot, int buf) {
#pragma unroll
      for (int u = 0; u < XU / 2; ++u) {
        const f32x4 lo = rx[slot][2 * u], hi = rx[slot][2 * u + 1];
        const u32x4 h = {pk_f16(lo.x, lo.y), pk_f16(lo.z, lo.w), pk_f16(hi.x, hi.y),
                         pk_f16(hi.z, hi.w)};
        *reinterpret_cast<u32x4*>(&As[buf][xb][(xr >> 4) + 2 * u][xe]) = h;
      }
      // block 0 decoded here into operand order; block 1 stays raw and is
      // decoded by the multiplying waves
      const uint32_t* c = rw[slot];
      f16x8* bw = &Bs[buf][tp >> 4][tp & 15];
#pragma unroll
      for (int g = 0; g < 4; ++g) bw[16 * g] = decode8_f16(shift16(c[g + 1], c[g]), c[0] & 0xFFFFu);
      *reinterpret_cast<u32x4*>(&Wc[buf][tp * 4]) = u32x4{c[5], c[6], c[7], c[8]};
      Wsc[buf][tp] = static_cast<uint16_t>(c[4] >> 16);
    };

    // step t: issue the loads of stage t + D into the register set stage t
    // used; put stage t + 1 into LDS buffer (t + 1) % 2 while the multiplying
    // waves read buffer t % 2 (stage s lives in register set s % D).
#define Q4_WSSTEP(I)                                 \
  do {                                               \
    load(t + (I) + WS_D, (I) % WS_D);                \
    __builtin_amdgcn_sched_barrier(0);               \
    if (t + (I) + 1 < nst)                           \
      store(((I) + 1) % WS_D, (t + (I) + 1) & 1);    \
    __syncthreads();                                 \
  } while (0)

#pragma unroll
    for (int i = 0; i < WS_D; ++i) load(i, i);
    store(0, 0);
    __syncthreads();
    int t = 0;
    for (; t + WS_D <= nst; t += WS_D) {
#pragma unroll
      for (int I = 0; I < WS_D; ++I) Q4_WSSTEP(I);
    }
#pragma unroll
    for (int I = 0; I < WS_D - 1; ++I)
      if (t + I < nst) Q4_WSSTEP(I);
#undef Q4_WSSTEP
  }
}

template <int BM>
__global__ __launch_bounds__(WS_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void matmul_ws_kernel(const uint8_t* __restrict__ W, const float* __restrict__ X,
                      float* __restrict__ Y, float* __restrict__ P, int M, int N, int K,
                      int tiles_n, int ntiles, int split_stages) {
  ws_body<BM, false>(W, X, Y, P, nullptr, M, N, K, tiles_n, ntiles, split_stages);
}

// Y = R + X deq(W)^T without a K split; R may be Y.
template <int BM>
__global__ __launch_bounds__(WS_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void matmul_ws_res_kernel(const uint8_t* __restrict__ W, const float* __restrict__ X, float* Y,
                          const float* R, int M, int N, int K, int tiles_n, int ntiles,
                          int split_stages) {
  ws_body<BM, true>(W, X, Y, nullptr, R, M, N, K, tiles_n, ntiles, split_stages);
}

// ---------------------------------------------------------------------------
// Skinny kernel: M <= 16 MT rows of X (MT <= 3), K % 64 == 0.  The decoder's
// prompt prefix (16 / 38 / 76 tokens) is far below a 128-row tile, and the
// product is bound by streaming W; so W is the MFMA A operand (16 weight rows
// per wave, decoded straight into operand registers) and X^T the B operand,
// shared by the 8 waves of a workgroup (128 weight rows) through LDS.  A
// stage is SK_PP block pairs: the workgroup stages the raw codes of its 128
// rows and the binary16 X^T of the stage (coalesced loads, a ring of SK_D
// register sets), then every wave decodes its rows and multiplies against all
// MT tiles of X; one barrier per stage.  Up to 32 rows of X a stage is 4
// pairs (256 k), beyond that 2 (LDS): stages of one pair were bound by the
// per-stage chain (LDS store, barrier, LDS read, decode, MFMA).  The last
// stage of a row may be partial; its missing pairs are skipped (all their
// loads are range-checked).
// Output lane layout of the 16 x 16 tile: C[n][m] with m = lane % 16 and
// n = 4 (lane / 16) + v, so each lane writes 4 consecutive columns of Y.
// ---------------------------------------------------------------------------
constexpr int SK_ROWS = 128, SK_THREADS = 512;
constexpr int SK_MAX_MT = 3;
// Rows of x up to which q4_matmul routes to the skinny kernel (its three
// tiles of 16 rows; it once served up to 80).  Past 48 rows the wide kernel's planner won on
// the decoder shapes (same box, 76 rows: QKV 17.0 vs 18.3 us, O 14.7 vs
// 16.0, gate+up 25.6 vs 32.0, down 20.6 vs 22.1); at 38 rows the skinny
// kernel was ahead or within 2 %.
constexpr int SK_ROUTE_MAX_M = 16 * SK_MAX_MT;
// Block pairs per stage: 4 up to 32 rows of X; beyond that the binary16 X^T
// of 4 pairs would leave one workgroup per CU (LDS), so 2.  A ring of two
// register sets.
constexpr int sk_pp(int mt) { return mt <= 2 ? 4 : 2; }
constexpr int SK_D = 2;

template <int MT>
__global__ __launch_bounds__(SK_THREADS) void matmul_skinny_kernel(
    const uint8_t* __restrict__ W, const float* __restrict__ X, float* __restrict__ Y,
    float* __restrict__ P, int M, int N, int K, int groups, int split_stages) {
  constexpr int SK_PP = sk_pp(MT);
  constexpr int SK_RD = SK_PP * 9;                          // code dwords per row and stage
  constexpr int SK_WDW = SK_ROWS * SK_RD;                   // code dwords per stage
  constexpr int SK_WU = (SK_WDW + SK_THREADS - 1) / SK_THREADS;
  constexpr bool WFULL = SK_WU * SK_THREADS == SK_WDW;      // else the last round is partial
  constexpr int XC = MT * 16 * 16 * SK_PP;                  // 16-byte X chunks per stage
  constexpr int XU = (XC + SK_THREADS - 1) / SK_THREADS;    // per thread
  __shared__ f16x8 Xs[2][SK_PP][2][MT][64];      // [buf][pair][block][m tile][element]
  __shared__ uint32_t Wraw[2][SK_WDW];

  const int item = xcd_tile(blockIdx.x, gridDim.x);
  const int split = item / groups, grp = item % groups;
  const int n0 = grp * SK_ROWS;
  const int nbp = K >> 6;
  const int nss = (nbp + SK_PP - 1) / SK_PP;    // stages in a row
  const int s0 = split * split_stages;
  const int nst = min(nss - s0, split_stages);  // >= 1 (host guarantees)
  const int64_t rb = static_cast<int64_t>(nbp) * PAIR_BYTES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // X staging: chunk c = tid + 512 u, q = c / 16: pair q / (16 MT), m tile
  // (q / 16) % MT, row in the tile spread so that the 4 rows of one wave's
  // store are one quad apart (its 8-byte destinations then hit every LDS
  // bank twice); 16-byte slot c % 16 of the pair.  Same operand order and
  // swizzle as the tile kernels: slot g of row r (block b) at element
  // 16 g + (r % 16 ^ (g + 4 b)).  Rows past M read as zeros.
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(X, static_cast<int64_t>(M) * K * 4);
  int xvo[XU], xlds[XU];
  bool xon[XU];
#pragma unroll
  for (int u = 0; u < XU; ++u) {
    const int c = tid + SK_THREADS * u;
    xon[u] = c < XC;  // wave-uniform
    const int q = c >> 4, jj = c & 15, qq = q & 15;
    const int mt = (q >> 4) % MT, pr = (q >> 4) / MT;
    const int rl = ((qq & 3) << 2) | (qq >> 2);
    const int r = 16 * mt + rl;
    const int xb = jj >> 3, xh = (jj >> 2) & 1, xg = jj & 3;
    xvo[u] = r * K * 4 + (16 * pr + jj) * 16;
    xlds[u] = (((pr * 2 + xb) * MT + mt) * 64 + 16 * xg + (rl ^ (xg + 4 * xb))) * 16 + 8 * xh;
  }
  // W staging: flat code dword f = tid + 512 u of the stage (row f / SK_RD,
  // dword f % SK_RD of the row's SK_PP pairs, contiguous in memory)
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(W + static_cast<int64_t>(n0) * rb,
                                               static_cast<int64_t>(N - n0) * rb);
  int wvo[SK_WU];
#pragma unroll
  for (int u = 0; u < SK_WU; ++u) {
    const int f = tid + SK_THREADS * u;
    wvo[u] = static_cast<int>((f / SK_RD) * rb) + (f % SK_RD) * 4;
  }
  const bool wlast = WFULL || tid < SK_WDW - (SK_WU - 1) * SK_THREADS;  // wave-uniform

  f32x4 rx[SK_D][XU];
  uint32_t rw[SK_D][SK_WU];
  // the stage offset goes into the range-checked vector offset: a partial
  // last stage reads past its row, and past the buffer for the last row
  auto load = [&](int t, int slot) {
    const int st = s0 + (t < nst ? t : nst - 1);
#pragma unroll
    for (int u = 0; u < XU; ++u)
      if (xon[u])
        rx[slot][u] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xvo[u] + st * (SK_PP * 256), 0, 0));
#pragma unroll
    for (int u = 0; u < SK_WU - 1; ++u)
      rw[slot][u] = __builtin_amdgcn_raw_buffer_load_b32(wrs, wvo[u] + st * (SK_PP * PAIR_BYTES), 0, 0);
    if (wlast)
      rw[slot][SK_WU - 1] = __builtin_amdgcn_raw_buffer_load_b32(
          wrs, wvo[SK_WU - 1] + st * (SK_PP * PAIR_BYTES), 0, 0);
  };
  // ordering guard (see the tile kernels): volatile first ops on loaded data
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
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  auto store = [&](int slot, int buf) {
#pragma unroll
    for (int u = 0; u < XU; ++u)
      if (xon[u]) {
        const f32x4 v = rx[slot][u];
        const u32x2 h = {pk_f16(v.x, v.y), pk_f16(v.z, v.w)};
        *reinterpret_cast<u32x2*>(reinterpret_cast<char*>(&Xs[buf][0][0][0][0]) + xlds[u]) = h;
      }
#pragma unroll
    for (int u = 0; u < SK_WU - 1; ++u) Wraw[buf][tid + SK_THREADS * u] = pin(rw[slot][u]);
    if (wlast) Wraw[buf][tid + SK_THREADS * (SK_WU - 1)] = pin(rw[slot][SK_WU - 1]);
  };

  // this wave's rows: n0 + 16 wave + lane % 16; lane group g = lane / 16.
  // Even and odd pairs accumulate separately (two MFMA chains).
  const int nl = lane & 15, g = lane >> 4;
  const int wbase = (16 * wave + nl) * SK_RD;
  const int xe0 = 16 * g + (nl ^ g), xe1 = 16 * g + (nl ^ (g + 4));
  f32x4v acc[2][MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[0][i] = acc[1][i] = f32x4v{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, int t) {
    const int pv = min(SK_PP, nbp - (s0 + t) * SK_PP);  // pairs present (uniform)
    const uint32_t* wr = &Wraw[buf][wbase];
#pragma unroll
    for (int p = 0; p < SK_PP; ++p) {
      if (p < pv) {
        const uint32_t* w9 = wr + 9 * p;
        const uint32_t q0a = w9[g], q0b = w9[g + 1], d01 = w9[0], d1w = w9[4], q1 = w9[5 + g];
        const f16x8 a0 = decode8_f16(shift16(q0b, q0a), d01 & 0xFFFFu);
        const f16x8 a1 = decode8_f16(q1, d1w >> 16);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          acc[p & 1][i] =
              __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, Xs[buf][p][0][i][xe0], acc[p & 1][i], 0, 0, 0);
          acc[p & 1][i] =
              __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, Xs[buf][p][1][i][xe1], acc[p & 1][i], 0, 0, 0);
        }
      }
    }
  };

  // Step t: issue the loads of stage t + D into the register set stage t
  // used; stage t + 1 (loaded D - 1 steps ago) into LDS buffer (t + 1) % 2;
  // multiply stage t from buffer t % 2; barrier.
#define Q4_SSTEP(I)                                         \
  do {                                                      \
    load(t + (I) + SK_D, (I) % SK_D);                       \
    __builtin_amdgcn_sched_barrier(0);                      \
    store(((I) + 1) % SK_D, ((I) + 1) % 2);                 \
    compute((I) % 2, t + (I));                              \
    __syncthreads();                                        \
  } while (0)

  static_assert(SK_D == 2, "the step is unrolled for a ring of two register sets");
  load(0, 0);
  load(1, 1);
  store(0, 0);
  __syncthreads();
  int t = 0;
  for (; t + 2 <= nst; t += 2) {
    Q4_SSTEP(0); Q4_SSTEP(1);
  }
  if (t < nst) Q4_SSTEP(0);
#undef Q4_SSTEP

  // Y[m][n] for m = 16 i + lane % 16, n = n0 + 16 wave + 4 (lane / 16) + v
  float* out = P ? P + static_cast<int64_t>(split) * M * N : Y;
  const int nb = n0 + 16 * wave + 4 * g;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int m = 16 * i + nl;
    if (m >= M) continue;
    const f32x4v a = acc[0][i] + acc[1][i];
    float* yr = out + static_cast<int64_t>(m) * N + nb;
    if ((N & 3) == 0 && nb + 4 <= N) {
      *reinterpret_cast<f32x4v*>(yr) = a;
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (nb + v < N) yr[v] = a[v];
    }
  }
}

// Y = sum over s of P[s] in the order s = 0, 1, ... (deterministic).  A
// thread requests all S of its slices before the first add: the slices were
// just written by workgroups on every XCD, so each read goes out to memory,
// and a chain of dependent load-then-add steps would pay that latency once
// per slice (measured ~4 us per call on the prefix shapes, mostly waiting).
// RES: Y = R + the sum (R may be Y itself); with S == 1 it is the
// residual add alone (P the product).
template <int S, bool RES>
__global__ __launch_bounds__(256) void splitk_fold_kernel(const float* __restrict__ P, float* Y,
                                                          const float* R, int64_t mn) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  if ((mn & 3) == 0) {
    const int64_t n4 = mn >> 2;
    const f32x4* p4 = reinterpret_cast<const f32x4*>(P);
    f32x4* y4 = reinterpret_cast<f32x4*>(Y);
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride) {
      f32x4 v[S];
#pragma unroll
      for (int s = 0; s < S; ++s) v[s] = p4[i + s * n4];
      f32x4 a = v[0];
#pragma unroll
      for (int s = 1; s < S; ++s) a += v[s];
      if constexpr (RES) a += reinterpret_cast<const f32x4*>(R)[i];
      y4[i] = a;
    }
  } else {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < mn; i += stride) {
      float v[S];
#pragma unroll
      for (int s = 0; s < S; ++s) v[s] = P[i + s * mn];
      float a = v[0];
#pragma unroll
      for (int s = 1; s < S; ++s) a += v[s];
      if constexpr (RES) a += R[i];
      Y[i] = a;
    }
  }
}

template <int S>
void launch_fold(const float* P, float* y, const float* r, int64_t mn, int splits, int blocks,
                 hipStream_t s) {
  if constexpr (S <= MAX_SPLITS) {
    if (splits == S) {
      if (r)
        hipLaunchKernelGGL((splitk_fold_kernel<S, true>), dim3(blocks), dim3(256), 0, s, P, y, r, mn);
      else
        hipLaunchKernelGGL((splitk_fold_kernel<S, false>), dim3(blocks), dim3(256), 0, s, P, y, r, mn);
      return;
    }
    launch_fold<S + 1>(P, y, r, mn, splits, blocks, s);
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

// Kernel and K-split plan for a shape.
enum MatmulKind { MM_STREAM, MM_SMALL, MM_STREAM16, MM_SKINNY, MM_WIDE, MM_WIDE96, MM_WIDE64, MM_WIDE32, MM_TILE, MM_SIMPLE };
struct MatmulPlan {
  MatmulKind kind;
  int splits;  // >= 1
  int stages;  // kernel stages per split (64 k; 128 or 256 k for the skinny kernel)
};

// Up to 4 rows of x (decode streams) keep the float32 accuracy of q4_matvec.
// Three or four rows with K <= 6144 take the stream16 kernel with x in two
// binary16 parts (measured 16 % faster per decoder layer than the routes
// below), and so do two rows with K <= 3072 over 20 MiB of weights or more.
// The matvec kernel (one set of workgroups per pair of rows of x,
// each weight read once per pair) serves one or two rows, any K % 64 == 32
// and the shapes whose repeated weight reads stay in the caches ((M - 1) *
// weight bytes up to STREAM_REREAD: measured faster there, it has no split
// and no fold launch); the small-M MFMA kernel, weights read once, the rest.
// 5 to 16 rows with K <= 6144, or up to 48 rows with K <= 3072: the
// stream16 kernel, weights read once by persistent workgroups that split K
// over their waves (measured 7-17 % faster per decoder layer than the
// skinny kernel, which pays per-stage costs, partial sums and a fold).
// Skinny for the other prompt-prefix shapes (bound by streaming W);
// 128 x 256 wave-specialised tiles for wide outputs (half the X traffic per
// flop of 128 x 128); 128 x 128 tiles otherwise.  K is split when the units
// alone cannot fill every workgroup slot: at least `min_st` stages per split,
// at most MAX_SPLITS, for the skinny kernel no more partial bytes than weight
// bytes, and never more than the workspace holds.
constexpr int64_t STREAM_REREAD = int64_t{40} << 20;
constexpr int64_t STREAM16_TWO_ROWS = int64_t{20} << 20;
static MatmulPlan plan_matmul(int64_t M, int64_t N, int64_t K, int cus, size_t ws_bytes) {
  if (M <= 4) {
    // three or four rows, K <= 6144: the stream16 kernel with x in two
    // binary16 parts (the q4_matvec bound), weights read once
    if (M >= 3 && matmul_stream16_chunks(M, K) > 0) return MatmulPlan{MM_STREAM16, 1, 0};
    const int64_t wbytes = N * (K / 32) * 18;
    // two rows, K <= 3072, 20 MiB of weights or more: the same (measured
    // against the pair kernel, same box, us: 12288 x 3072 9.4 / 10.1,
    // 18432 x 3072 11.7 / 12.9, 131072 x 3072 49.0 / 58.2; below 20 MiB and
    // for longer rows the pair kernel is as fast or faster)
    if (M == 2 && K <= 3072 && wbytes >= STREAM16_TWO_ROWS && matmul_stream16_chunks(M, K) > 0)
      return MatmulPlan{MM_STREAM16, 1, 0};
    if (M == 1 || K % 64 != 0 || (K <= 12288 && (M == 2 || (M - 1) * wbytes <= STREAM_REREAD)))
      return MatmulPlan{MM_STREAM, 1, 0};
  }
  if (K % 64 != 0) return MatmulPlan{MM_SIMPLE, 1, 0};
  if (matmul_stream16_chunks(M, K) > 0) return MatmulPlan{MM_STREAM16, 1, 0};
  const int nbp = static_cast<int>(K / 64);
  MatmulKind kind;
  int64_t units, slots, min_st, cap = MAX_SPLITS;
  if (M <= 4) {
    kind = MM_SMALL;
    units = (N + 63) / 64;
    // one round, never a partial second: all resident workgroups when the
    // 64-row groups fill half the GPU, else one per CU (fewer, longer splits
    // measured faster there, as for the skinny kernel)
    slots = (2 * units > cus ? static_cast<int64_t>(matmul_small_per_cu()) : 1) *
            static_cast<int64_t>(cus);
    min_st = 4;
  } else if (M <= SK_ROUTE_MAX_M) {
    kind = MM_SKINNY;
    units = (N + SK_ROWS - 1) / SK_ROWS;
    // one workgroup per CU, two when the row groups alone fill half the CUs
    // (measured on the prefix shapes: fewer, longer splits win for N <= 6144,
    // more workgroups for the 18432-row gate+up)
    slots = (2 * units > cus ? 2 : 1) * static_cast<int64_t>(cus);
    min_st = 4 / sk_pp(static_cast<int>((M + 15) / 16));  // at least 256 k per split
    cap = std::max<int64_t>(1, (K * 9 / 16) / (4 * M));
  } else if (N >= 512) {
    kind = MM_WIDE;
    units = ((M + T_BM - 1) / T_BM) * ((N + WS_BN - 1) / WS_BN);
    slots = cus;
    min_st = 4;
  } else {
    kind = MM_TILE;
    units = ((M + T_BM - 1) / T_BM) * ((N + 127) / 128);
    slots = 2 * static_cast<int64_t>(cus);
    min_st = 8;
  }
  // stages of the kernel: sk_pp pairs for the skinny kernel, one pair otherwise
  const int spp = kind == MM_SKINNY ? sk_pp(static_cast<int>((M + 15) / 16)) : 1;
  const int nstg = (nbp + spp - 1) / spp;
  const int64_t slice = M * N * static_cast<int64_t>(sizeof(float));
  int64_t want;
  if (kind == MM_WIDE) {
    // Estimated time (us) of (M tile, S splits): the stages of the busiest
    // workgroup slot, plus (S > 1) the partial slices and a fixed cost per
    // split call.  Fitted to encoder-shape timings: 0.92 us per 128 x 256 x 64
    // stage, 0.85 us per 96-row, 0.7 us per 64-row, 0.55 us per 32-row stage,
    // 0.33 us per MB of partial slices (written, then read back by the fold)
    // and 4 us for the fold's launch and the shorter pipelines.  The shorter
    // tiles win where the taller ones leave CUs idle (the 1280-wide
    // projections, M <= 375); K is split for few tiles and long K.
    want = 1;
    double best = -1.0;
    const int64_t smax = std::min<int64_t>(MAX_SPLITS, nstg);
    const int64_t tn = (N + WS_BN - 1) / WS_BN;
    const struct { MatmulKind k; int64_t u; double ts; } opt[4] = {
        {MM_WIDE, ((M + 127) / 128) * tn, 0.92}, {MM_WIDE96, ((M + 95) / 96) * tn, 0.85},
        {MM_WIDE64, ((M + 63) / 64) * tn, 0.7}, {MM_WIDE32, ((M + 31) / 32) * tn, 0.55}};
    for (const auto& o : opt) {
      for (int64_t sp = 1; sp <= smax; ++sp) {
        if (sp > 1 && static_cast<uint64_t>(sp * slice) > ws_bytes) break;
        // prompt prefixes (HBM bound): no more partial bytes than weight
        // bytes, the skinny kernel's rule (the model alone chose 96-row
        // tiles split 8 for QKV at 76 rows, 19.2 us, where 64-row tiles
        // split 5 measured 17.0)
        if (sp > 1 && M <= 80 && sp * slice > N * (K / 32) * 18) break;
        const int64_t per = (nstg + sp - 1) / sp;
        const int64_t rounds = (o.u * sp + slots - 1) / slots;
        double est = o.ts * static_cast<double>(per * rounds);
        if (sp > 1) est += 3.3e-7 * static_cast<double>(sp * slice) + 4.0;
        if (best < 0.0 || est < best) {
          best = est;
          want = sp;
          kind = o.k;
        }
      }
    }
  } else {
    want = slots / units;
    want = std::min<int64_t>(want, nstg / min_st);
    want = std::min<int64_t>(want, std::min<int64_t>(cap, MAX_SPLITS));
    while (want > 1 && static_cast<uint64_t>(want * slice) > ws_bytes) --want;
  }
  if (want < 2) return MatmulPlan{kind, 1, nstg};
  int per = static_cast<int>((nstg + want - 1) / want);
  if (kind == MM_SMALL) per = (per + 3) & ~3;  // whole 4-pair chunks per split
  return MatmulPlan{kind, (nstg + per - 1) / per, per};  // every split non-empty
}

const char* matmul_route(int64_t M, int64_t N, int64_t K, size_t ws_bytes, int cus, int* splits) {
  const MatmulPlan p = plan_matmul(M, N, K, cus, ws_bytes);
  if (splits) *splits = p.splits;
  switch (p.kind) {
    case MM_STREAM: return "matvec";
    case MM_SMALL: return "small";
    case MM_STREAM16: return "stream16";
    case MM_SKINNY: return "skinny";
    case MM_WIDE: return "wide128";
    case MM_WIDE96: return "wide96";
    case MM_WIDE64: return "wide64";
    case MM_WIDE32: return "wide32";
    case MM_TILE: return "tile";
    case MM_SIMPLE: return "simple";
  }
  return "unknown";
}

size_t matmul_workspace_bytes(int64_t M, int64_t N, int64_t K, int cus) {
  const MatmulPlan p = plan_matmul(M, N, K, cus, SIZE_MAX);
  return p.splits > 1 ? static_cast<size_t>(p.splits) * M * N * sizeof(float) : 0;
}

template <int BN, int D>
static void launch_tile(const uint8_t* w, const float* x, float* y, float* P, int64_t M,
                        int64_t N, int64_t K, int splits, int stages, hipStream_t s) {
  const int tiles_n = static_cast<int>((N + BN - 1) / BN);
  const int tiles_m = static_cast<int>((M + T_BM - 1) / T_BM);
  const int ntiles = tiles_n * tiles_m;
  hipLaunchKernelGGL((matmul_tile_kernel<BN, D>), dim3(ntiles * splits),
                     dim3(TileCfg<BN>::THREADS), 0, s, w, x, y, P, static_cast<int>(M),
                     static_cast<int>(N), static_cast<int>(K), tiles_n, ntiles, stages);
}

template <int MT>
static void launch_skinny(const uint8_t* w, const float* x, float* y, float* P, int64_t M,
                          int64_t N, int64_t K, int splits, int stages, hipStream_t s) {
  const int groups = static_cast<int>((N + SK_ROWS - 1) / SK_ROWS);
  hipLaunchKernelGGL((matmul_skinny_kernel<MT>), dim3(groups * splits), dim3(SK_THREADS), 0, s,
                     w, x, y, P, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K),
                     groups, stages);
}

template <int BM>
static void launch_ws(const uint8_t* w, const float* x, float* y, float* P, const float* r,
                      int64_t M, int64_t N, int64_t K, int splits, int stages, hipStream_t s) {
  const int tiles_n = static_cast<int>((N + WS_BN - 1) / WS_BN);
  const int ntiles = tiles_n * static_cast<int>((M + BM - 1) / BM);
  // the residual rides in these stores only without a K split (else in the fold)
  if (r != nullptr && P == nullptr)
    hipLaunchKernelGGL(matmul_ws_res_kernel<BM>, dim3(ntiles), dim3(WS_THREADS), 0, s, w, x, y, r,
                       static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), tiles_n,
                       ntiles, stages);
  else
    hipLaunchKernelGGL(matmul_ws_kernel<BM>, dim3(ntiles * splits), dim3(WS_THREADS), 0, s, w, x, y,
                       P, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), tiles_n,
                       ntiles, stages);
}

static bool is_wide(MatmulKind k) {
  return k == MM_WIDE || k == MM_WIDE96 || k == MM_WIDE64 || k == MM_WIDE32;
}

// Whether Y = R + product adds R inside a kernel of the product: in the
// wide kernel's stores (no K split) or in the fold (any K split); else a
// second launch adds it to the finished product.
static bool residual_fused(const MatmulPlan& p) { return p.splits > 1 || is_wide(p.kind); }

bool matmul_residual_fused(int64_t M, int64_t N, int64_t K, size_t ws_bytes, int cus) {
  return residual_fused(plan_matmul(M, N, K, cus, ws_bytes));
}

size_t matmul_residual_workspace_bytes(int64_t M, int64_t N, int64_t K, int cus) {
  const MatmulPlan p = plan_matmul(M, N, K, cus, SIZE_MAX);
  const size_t split = p.splits > 1 ? static_cast<size_t>(p.splits) * M * N * sizeof(float) : 0;
  // in place on an unfused route the product waits in the workspace
  const size_t temp = residual_fused(p) ? 0 : static_cast<size_t>(M) * N * sizeof(float);
  return std::max(split, temp);
}

hipError_t launch_matmul(const uint8_t* w, const float* x, float* y, const float* r, int64_t M,
                         int64_t N, int64_t K, void* ws, size_t ws_bytes, int cus, hipStream_t s) {
  const MatmulPlan p = plan_matmul(M, N, K, cus, ws ? ws_bytes : 0);
  if (p.splits > MAX_SPLITS) return hipErrorInvalidValue;  // the planner caps it; the fold relies on it
  const int64_t mn = M * N;
  auto fold_blocks = [&]() {
    const int64_t items = (mn & 3) == 0 ? mn / 4 : mn;
    return static_cast<int>(std::min<int64_t>((items + 255) / 256, 4 * cus));
  };
  if (r != nullptr && !residual_fused(p)) {
    // No K split, so the product kernel leaves the workspace alone: in place
    // (R is Y) the product goes there, else straight to Y; then Y = R + it.
    float* dst = r == y ? static_cast<float*>(ws) : y;
    if (dst == nullptr || (r == y && ws_bytes < static_cast<size_t>(mn) * sizeof(float)))
      return hipErrorInvalidValue;  // the entry point checks this first
    const hipError_t e = launch_matmul(w, x, dst, nullptr, M, N, K, ws, ws_bytes, cus, s);
    if (e != hipSuccess) return e;
    launch_fold<1>(dst, y, r, mn, 1, fold_blocks(), s);
    return hipGetLastError();
  }
  float* P = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
  switch (p.kind) {
    case MM_STREAM:
      return launch_matvec(w, x, y, M, N, K, s);
    case MM_SMALL:
      launch_matmul_small(w, x, y, P, M, N, K, p.splits, p.stages, s);
      break;
    case MM_STREAM16:
      return launch_matmul_stream16(w, x, y, M, N, K, cus, s);
    case MM_SKINNY:
      switch ((M + 15) / 16) {
        case 1: launch_skinny<1>(w, x, y, P, M, N, K, p.splits, p.stages, s); break;
        case 2: launch_skinny<2>(w, x, y, P, M, N, K, p.splits, p.stages, s); break;
        default: launch_skinny<3>(w, x, y, P, M, N, K, p.splits, p.stages, s); break;
      }
      break;
    case MM_WIDE:
      launch_ws<128>(w, x, y, P, r, M, N, K, p.splits, p.stages, s);
      break;
    case MM_WIDE96:
      launch_ws<96>(w, x, y, P, r, M, N, K, p.splits, p.stages, s);
      break;
    case MM_WIDE64:
      launch_ws<64>(w, x, y, P, r, M, N, K, p.splits, p.stages, s);
      break;
    case MM_WIDE32:
      launch_ws<32>(w, x, y, P, r, M, N, K, p.splits, p.stages, s);
      break;
    case MM_TILE:
      launch_tile<128, 3>(w, x, y, P, M, N, K, p.splits, p.stages, s);
      break;
    case MM_SIMPLE: {
      const dim3 grid(static_cast<unsigned>((N + S_BN - 1) / S_BN),
                      static_cast<unsigned>((M + S_BM - 1) / S_BM));
      hipLaunchKernelGGL(matmul_simple_kernel, grid, dim3(S_THREADS), 0, s, w, x, y,
                         static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
      break;
    }
  }
  if (p.splits > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_fold<2>(P, y, r, mn, p.splits, fold_blocks(), s);
  }
  return hipGetLastError();
}

}  // namespace q4
