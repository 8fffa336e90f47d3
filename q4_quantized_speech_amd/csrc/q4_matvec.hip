// Q4_0 matrix-vector product (decode step) and the LM-head argmax.
//
// Section "Architecture" of "Implémentation en Rust du modèle Voxtral Mini 4B
// Realtime de Mistral pour l'exécuter dans le navigateur": every decoder
// projection runs on Q4_0 weights; per generated token each weight byte is read
// once, so this kernel is an HBM stream.  Design for gfx950:
//  * a row is read as 36-byte block pairs (two Q4_0 blocks; with K % 64 == 0
//    every pair is dword aligned).  16 lanes cover 16 consecutive pairs of a
//    row (576 contiguous bytes per DPP row); the K range is split over
//    KS = ceil(K / 1024) waves of the workgroup, so every lane owns exactly one
//    pair column for the whole kernel;
//  * that lane keeps its 64 x values in registers (the high nibbles' x
//    divided by 16, exact).  Each wave reads its 1024-float slice of x once,
//    coalesced (16 B per lane per load), and hands every lane its 64 values
//    through LDS: loading them straight from memory would touch 16 cache
//    lines per load instruction, which costs more address-unit time at the
//    start of a workgroup than a pass of weights;
//  * x is requested before the weights and the first two passes of weights
//    right after, so waiting for x never waits for weights (the memory
//    counter is in order) and two passes are in flight from the start;
//  * each lane serves R = 2 rows per pass (4 DPP rows per wave -> 8 rows), or
//    R = 1 where the finer passes spread a short matrix over more CUs;
//    passes are double-buffered with two register sets used alternately, so
//    the in-order vmcnt counter lets the next pass's loads fly while the
//    current one computes; rows are read through a range-checked buffer
//    resource based at the pass's first row;
//  * codes become centred binary16 values (q - 8, the high nibbles in place
//    as 16 (q - 8) against x / 16; one mask-and-insert under the exponent of
//    1024 and one packed add per two codes, exact) fed to v_fma_mix, which
//    converts and multiply-adds in one instruction per weight; the two
//    blocks' chains are interleaved so no FMA waits on the one before it.
//    Per block, y += d * sum_j (q_j - 8) x_j: every rounding is relative to
//    sum |w x|, whatever the spread of x;
//  * the 16 lanes of a row are summed in their DPP row, the KS waves' partial
//    sums are then added in LDS in a fixed order (deterministic results);
//  * workgroups are persistent (a grid-stride loop over row groups), as many
//    as are resident at once, with the passes spread evenly over them;
//  * with two or more rows of x, a workgroup takes them in pairs: the codes
//    are loaded and decoded once and feed each row's own chains, in the
//    order of the one-row kernel (every row keeps the bits it has alone).
// The argmax variant (the LM head over the 131072-row table that section
// "Solutions techniques", item 3, keeps in Q4) tracks the best (value, lowest
// index) per lane, reduces it per workgroup, and folds it into a per-row key
// in the workspace with one device-scope atomic max; the last workgroup to
// arrive writes the result and clears the workspace (no second launch).

#include <atomic>
#include <mutex>

#include "q4_device.h"
#include "q4_kernels.h"

namespace q4 {
namespace {



// Eight codes of one qs dword against x (low nibbles) and x/16 (high
// nibbles), for two dwords at once.  Each code goes into a half-word under
// the binary16 exponent of 1024 (0x6400 | n, n the low nibble or 16 times the
// high one) and one packed binary16 add of -1032 or -1152 leaves q - 8 or
// 16 (q - 8), exactly; v_fma_mix converts the half-word for free.  The sums
// are of (q - 8) x terms, so their rounding is relative to sum |w x| (an
// offset form, sum q x - 8 sum x, would lose that bound when a large x meets
// a zero weight).  The two chains are interleaved instruction by instruction:
// a v_fma_mix right after the one it depends on costs a wait state.
// `magic` is 0x64006400 held in a VGPR (the caller keeps it there), so each
// mask-and-insert is one v_and_or_b32 (a VOP3 takes at most one scalar
// constant).  With MX rows of x the codes are decoded once and multiplied
// into each row's own pair of chains.
template <int MX>
__device__ __forceinline__ void nib_dot8_mix2(uint32_t q0, uint32_t q1, const f32x4 (&xl0)[MX],
                                              const f32x4 (&xh0)[MX], const f32x4 (&xl1)[MX],
                                              const f32x4 (&xh1)[MX], float (&acc0)[MX],
                                              float (&acc1)[MX], uint32_t magic) {
  const f16x2 lo_off = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
  const f16x2 hi_off = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
  const uint32_t v0 = q0 >> 8, v1 = q1 >> 8;
  const f16x2 a0 = __builtin_bit_cast(f16x2, (q0 & 0x000F000Fu) | magic) + lo_off;
  const f16x2 a1 = __builtin_bit_cast(f16x2, (q1 & 0x000F000Fu) | magic) + lo_off;
  const f16x2 b0 = __builtin_bit_cast(f16x2, (q0 & 0x00F000F0u) | magic) + hi_off;
  const f16x2 b1 = __builtin_bit_cast(f16x2, (q1 & 0x00F000F0u) | magic) + hi_off;
  const f16x2 c0 = __builtin_bit_cast(f16x2, (v0 & 0x000F000Fu) | magic) + lo_off;
  const f16x2 c1 = __builtin_bit_cast(f16x2, (v1 & 0x000F000Fu) | magic) + lo_off;
  const f16x2 e0 = __builtin_bit_cast(f16x2, (v0 & 0x00F000F0u) | magic) + hi_off;
  const f16x2 e1 = __builtin_bit_cast(f16x2, (v1 & 0x00F000F0u) | magic) + hi_off;
  // each row of x: its own two chains, in the same order whatever MX
#pragma unroll
  for (int i = 0; i < MX; ++i) {
    float s0 = acc0[i], s1 = acc1[i];
    s0 = __builtin_fmaf(static_cast<float>(a0.x), xl0[i].x, s0);
    s1 = __builtin_fmaf(static_cast<float>(a1.x), xl1[i].x, s1);
    s0 = __builtin_fmaf(static_cast<float>(c0.x), xl0[i].y, s0);
    s1 = __builtin_fmaf(static_cast<float>(c1.x), xl1[i].y, s1);
    s0 = __builtin_fmaf(static_cast<float>(a0.y), xl0[i].z, s0);
    s1 = __builtin_fmaf(static_cast<float>(a1.y), xl1[i].z, s1);
    s0 = __builtin_fmaf(static_cast<float>(c0.y), xl0[i].w, s0);
    s1 = __builtin_fmaf(static_cast<float>(c1.y), xl1[i].w, s1);
    s0 = __builtin_fmaf(static_cast<float>(b0.x), xh0[i].x, s0);
    s1 = __builtin_fmaf(static_cast<float>(b1.x), xh1[i].x, s1);
    s0 = __builtin_fmaf(static_cast<float>(e0.x), xh0[i].y, s0);
    s1 = __builtin_fmaf(static_cast<float>(e1.x), xh1[i].y, s1);
    s0 = __builtin_fmaf(static_cast<float>(b0.y), xh0[i].z, s0);
    s1 = __builtin_fmaf(static_cast<float>(b1.y), xh1[i].z, s1);
    s0 = __builtin_fmaf(static_cast<float>(e0.y), xh0[i].w, s0);
    s1 = __builtin_fmaf(static_cast<float>(e1.y), xh1[i].w, s1);
    acc0[i] = s0;
    acc1[i] = s1;
  }
}

// Argmax bookkeeping: idx < 0 means "no candidate", which never wins over a
// candidate, whatever its value; NaN never wins.
__device__ __forceinline__ bool am_better(float v, int i, float bv, int bi) {
  if (i < 0 || v != v) return false;
  if (bi < 0) return true;
  return v > bv || (v == bv && i < bi);
}

// Fold the candidates of all threads of the workgroup; result valid in thread 0.
// A butterfly over each wave, then one over the waves' candidates in wave 0:
// the order of a strict total order's comparisons does not change the winner.
__device__ __forceinline__ void am_block_reduce(float& bv, int& bi) {
  __shared__ float sv[16];
  __shared__ int si[16];
  auto fold = [&](int lanes) {
    for (int o = lanes >> 1; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, lanes);
      const int oi = __shfl_xor(bi, o, lanes);
      const bool t = am_better(ov, oi, bv, bi);
      bv = t ? ov : bv;
      bi = t ? oi : bi;
    }
  };
  fold(64);
  const int w = threadIdx.x >> 6, nw = static_cast<int>((blockDim.x + 63) >> 6);
  if ((threadIdx.x & 63) == 0) { sv[w] = bv; si[w] = bi; }
  __syncthreads();
  if (w == 0) {
    const int l = threadIdx.x;
    bv = l < nw ? sv[l] : 0.f;
    bi = l < nw ? si[l] : -1;
    fold(16);
  }
}

// Workspace layout, per row of x (256 bytes, key and counter on separate
// cache lines): a 64-bit key and a 32-bit arrival counter, both zero between
// calls.  key = order-preserving bits of the value (high word) | ~index (low
// word), so the largest key is the largest value with the lowest index, and
// 0 means "no candidate" (NaN never enters).  Each workgroup folds its
// candidate in with one device-scope atomic max, then counts itself in; the
// workgroup that arrives last takes an acquire fence, reads the key, writes
// the outputs and clears both words for the next call.
// Ordering, in the memory model's terms: a workgroup whose max raised the
// key (the max returns the old key) counts itself in with a release
// increment, which orders its max before its count; one whose max changed
// nothing has nothing to publish and counts itself in relaxed.  The
// increments all act on one counter, so every release heads a release
// sequence that the later increments continue, and the last workgroup's
// increment reads the end of it: its acquire fence synchronizes with every
// raising workgroup's release, and its read of the key sees at least every
// raised value -- the largest key among them is the largest of all (a
// workgroup whose max changed nothing saw a key at least as large, written
// by a raising one).  A release is an L2 writeback and an acquire an L2
// invalidation on this chip, each costing ~6 us on the 131072-row table when
// every workgroup took them; in arrival order only a few workgroups (about
// the logarithm of their number) raise the key.
constexpr int AM_ROW_BYTES = 256;
__device__ __forceinline__ uint64_t am_key(float v, int i) {
  if (i < 0 || v != v) return 0;
  if (v == 0.f) v = 0.f;  // -0 and +0 tie, like the comparisons above
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(o) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(i));
}
// The chosen token's row of the (tied) table, decoded by the whole
// workgroup: out[0..K) = deq(W[idx]), zeros when there is no candidate.
__device__ __forceinline__ void am_embed_row(const uint8_t* __restrict__ W, int idx, int64_t N,
                                             int K, float* __restrict__ out) {
  const int nb = K / QK;
  for (int b = static_cast<int>(threadIdx.x); b < nb; b += static_cast<int>(blockDim.x)) {
    f32x4* dst = reinterpret_cast<f32x4*>(out + static_cast<int64_t>(b) * QK);
    if (idx < 0 || idx >= N) {
#pragma unroll
      for (int u = 0; u < 8; ++u) dst[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      continue;
    }
    uint32_t d16, qs[4];
    load_block_any(W, static_cast<int64_t>(idx) * nb + b, d16, qs);
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
}

// emb (nullable): where the last workgroup of row m also writes the decoded
// table row of the chosen index (K floats at emb + m K), so the next decode
// step's input needs no second launch.
__device__ __forceinline__ void am_publish(float bv, int bi, int m, void* workspace, int nwg,
                                           int32_t* out_idx, float* out_val,
                                           const uint8_t* __restrict__ W, float* emb, int64_t N,
                                           int K) {
  __shared__ int s_chosen;  // the index, in the last workgroup; -2 in the others
  char* row = reinterpret_cast<char*>(workspace) + static_cast<int64_t>(m) * AM_ROW_BYTES;
  uint64_t* key = reinterpret_cast<uint64_t*>(row);
  uint32_t* count = reinterpret_cast<uint32_t*>(row + 128);
  am_block_reduce(bv, bi);
  if (threadIdx.x == 0) {
    s_chosen = -2;
    const uint64_t mine = am_key(bv, bi);
    const uint64_t old = __hip_atomic_fetch_max(key, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t prev;
    if (mine > old)
      prev = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    else
      prev = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == static_cast<uint32_t>(nwg - 1)) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      const uint64_t k = __hip_atomic_load(key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(key, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int idx = -1;
      float val = __builtin_nanf("");
      if (k != 0) {
        const uint32_t o = static_cast<uint32_t>(k >> 32);
        val = __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
        idx = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(k));
      }
      out_idx[m] = idx;
      if (out_val) out_val[m] = val;
      s_chosen = idx;
    }
  }
  if (emb != nullptr) {  // the same in every thread
    __syncthreads();
    const int idx = s_chosen;
    if (idx != -2) am_embed_row(W, idx, N, K, emb + static_cast<int64_t>(m) * K);
  }
}

// Pair kernel: K % 64 == 0, K <= 12288, KS = ceil(K / 1024) waves per workgroup.
// XL: x stays in LDS and is read every pass (56 VGPRs at R = 1: 8 waves per
// SIMD) instead of living in 64 registers per lane (4 waves per SIMD).
// G row groups of KS waves share the workgroup's x (each group stages a
// quarter of it when G = 4) and cover 4 R G consecutive rows per pass.
// MX rows of x per workgroup (1 or 2): the weights are read and decoded once
// for both rows; each row keeps its own chains in the one-row order, so its
// results have the bits it would have alone.  A missing second row (odd M)
// repeats the first and is never stored (nor published by the argmax).
template <int KS, bool ARGMAX, int R, bool XL, int G, int MX>
__global__ __launch_bounds__(64 * KS * G) void matvec_pairs_kernel(
    const uint8_t* __restrict__ W, const float* __restrict__ X, float* __restrict__ Y,
    int32_t* __restrict__ out_idx, float* __restrict__ out_val, void* workspace, int64_t N,
    int K, int M) {
  static_assert(MX == 1 || MX == 2, "one or two rows of x per workgroup");
  constexpr int ROWS = 4 * R * G;  // rows per pass
  __shared__ float red[2][KS][MX * ROWS];
  const int m = blockIdx.y * MX;  // first row of x
  int mr[MX];                     // the rows of x this workgroup reads
#pragma unroll
  for (int i = 0; i < MX; ++i) mr[i] = m + i < M ? m + i : m;
  const int nbp = K >> 6;
  const int64_t rb = static_cast<int64_t>(nbp) * PAIR_BYTES;
  const int tid = threadIdx.x;
  const int wv = tid >> 6, ks = wv % KS, gi = wv / KS, j = tid & 15;
  const int grp = gi * 4 + ((tid >> 4) & 3);  // DPP row of the pass
  const int craw = j + 16 * ks;
  const bool cvalid = craw < nbp;
  const int c = cvalid ? craw : nbp - 1;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * ROWS;

  // Weights of the first pass, then this lane's x slice (64 floats) and sums.
  // A pass's rows are read through a range-checked buffer resource based at
  // its first row (uniform), so each lane keeps constant offsets and rows past
  // N read as zeros (they are never stored).
  int64_t row0 = static_cast<int64_t>(blockIdx.x) * ROWS;
  uint32_t wa[R][9], wb[R][9];
  int wvo[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    wvo[r] = static_cast<int>((grp * R + r) * rb) + c * PAIR_BYTES;
  auto load = [&](int64_t r0, uint32_t (&w)[R][9]) {
    const int64_t left = N - r0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(W + (left > 0 ? r0 : 0) * rb), 0,
        left > 0 ? static_cast<int>((left < ROWS ? left : ROWS) * rb) : 0, 0x00020000);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, wvo[r], 0, 0));
      const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, wvo[r], 16, 0));
      w[r][0] = a.x; w[r][1] = a.y; w[r][2] = a.z; w[r][3] = a.w;
      w[r][4] = b.x; w[r][5] = b.y; w[r][6] = b.z; w[r][7] = b.w;
      w[r][8] = __builtin_amdgcn_raw_buffer_load_b32(rs, wvo[r], 32, 0);
    }
  };
  // x first (coalesced: the wave's 1024-float slice, 16 B per lane per load),
  // then the weights of the first two passes, so that waiting for x does not
  // wait for the weights; x goes to LDS (kept there, or copied to this lane's
  // registers), in rows of 64 floats padded to 68 so the 16 lanes of a DPP
  // row hit distinct banks.
  __shared__ float xs[MX][KS][16][68];
  f32x4 xg[MX][4];
#pragma unroll
  for (int i = 0; i < MX; ++i) {
    const float* xw = X + static_cast<int64_t>(mr[i]) * K + 1024 * ks;
    const int lim = K - 1024 * ks;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = (u * 64 + (tid & 63)) * 4;
      if (u % G == gi)
        xg[i][u] = p < lim ? *reinterpret_cast<const f32x4*>(xw + p) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  load(row0, wa);
  load(row0 + stride, wb);
  // x of the high nibbles is divided by 16 (exact) on the way in
#pragma unroll
  for (int i = 0; i < MX; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u % G != gi) continue;
      const int p = u * 64 + (tid & 63);
      f32x4 v = xg[i][u];
      if (p & 4) v *= 0.0625f;
      *reinterpret_cast<f32x4*>(&xs[i][ks][p >> 4][(p & 15) * 4]) = v;
    }
  }
  __syncthreads();
  float xv[MX][XL ? 1 : 64];
  if constexpr (!XL) {
#pragma unroll
    for (int i = 0; i < MX; ++i) {
      const float* xr = &xs[i][ks][j][0];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(xr + 4 * t);
        xv[i][4 * t] = v.x; xv[i][4 * t + 1] = v.y; xv[i][4 * t + 2] = v.z; xv[i][4 * t + 3] = v.w;
      }
    }
  }
  // the 16 x values of step t for row i: low and high nibbles of the two blocks
  auto xstep = [&](int i, int t, int xo, f32x4& xl0, f32x4& xh0, f32x4& xl1, f32x4& xh1) {
    if constexpr (XL) {
      const float* xr = &xs[i][ks][j][0];
      xl0 = *reinterpret_cast<const f32x4*>(xr + xo + 4 * t);
      xh0 = *reinterpret_cast<const f32x4*>(xr + xo + 16 + 4 * t);
      xl1 = *reinterpret_cast<const f32x4*>(xr + xo + 32 + 4 * t);
      xh1 = *reinterpret_cast<const f32x4*>(xr + xo + 48 + 4 * t);
    } else {
      const float* v = xv[i];
      xl0 = f32x4{v[4 * t], v[4 * t + 1], v[4 * t + 2], v[4 * t + 3]};
      xh0 = f32x4{v[16 + 4 * t], v[17 + 4 * t], v[18 + 4 * t], v[19 + 4 * t]};
      xl1 = f32x4{v[32 + 4 * t], v[33 + 4 * t], v[34 + 4 * t], v[35 + 4 * t]};
      xh1 = f32x4{v[48 + 4 * t], v[49 + 4 * t], v[50 + 4 * t], v[51 + 4 * t]};
    }
  };

  // scale bits of a lane past the last pair forced to +0 (a mask, not a
  // branch: a branch here lets the compiler split the rows of a pass apart)
  const uint32_t dmask = cvalid ? 0xFFFFu : 0u;
  uint32_t magic = 0x64006400u;  // binary16 1024 in both halves
  asm("" : "+v"(magic));
  // sum over this lane's pair for R rows of W and MX rows of x:
  // d0 * sum (q - 8) x + d1 * (...)
  auto compute = [&](uint32_t (&w)[R][9], float (&acc)[MX][R]) {
    int xo = 0;  // opaque per pass, so the LDS reads of x stay in the pass
    if constexpr (XL) asm volatile("" : "+v"(xo));
    float s0[R][MX], s1[R][MX];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < MX; ++i) s0[r][i] = s1[r][i] = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4 xl0[MX], xh0[MX], xl1[MX], xh1[MX];
#pragma unroll
      for (int i = 0; i < MX; ++i) xstep(i, t, xo, xl0[i], xh0[i], xl1[i], xh1[i]);
#pragma unroll
      for (int r = 0; r < R; ++r)
        nib_dot8_mix2<MX>(shift16(w[r][t + 1], w[r][t]), w[r][5 + t], xl0, xh0, xl1, xh1, s0[r],
                          s1[r], magic);
      // one step's x live at a time
      if constexpr (XL) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float d0 = half_bits_to_float(w[r][0] & dmask);
      const float d1 = half_bits_to_float((w[r][4] >> 16) & dmask);
#pragma unroll
      for (int i = 0; i < MX; ++i) acc[i][r] = __builtin_fmaf(d1, s1[r][i], d0 * s0[r][i]);
    }
  };

  float bv[MX];
  int bi[MX];
#pragma unroll
  for (int i = 0; i < MX; ++i) { bv[i] = 0.f; bi[i] = -1; }
  // Reduce the pass at r0 without branches: every lane of a DPP row holds the
  // row's sum (same bits) and writes it (same value, same address), every
  // wave adds the KS partial sums (LDS buffer q), then wave 0 consumes them:
  // a store through a resource covering this pass's rows of Y, with an
  // out-of-range offset for all lanes but one per row, or the argmax update
  // as selects.
  auto finish = [&](int64_t r0, float (&acc)[MX][R], int q) {
#pragma unroll
    for (int i = 0; i < MX; ++i)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[i][r] = row16_sum(acc[i][r]);
    if constexpr (KS > 1) {
#pragma unroll
      for (int i = 0; i < MX; ++i)
#pragma unroll
        for (int r = 0; r < R; ++r) red[q][ks][i * ROWS + grp * R + r] = acc[i][r];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MX; ++i) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float sum = red[q][0][i * ROWS + grp * R + r];
          for (int u = 1; u < KS; ++u) sum += red[q][u][i * ROWS + grp * R + r];
          acc[i][r] = sum;
        }
      }
    }
    if constexpr (ARGMAX) {
#pragma unroll
      for (int i = 0; i < MX; ++i) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int row = static_cast<int>(r0) + grp * R + r;
          const bool take = ks == 0 && row < N && am_better(acc[i][r], row, bv[i], bi[i]);
          bv[i] = take ? acc[i][r] : bv[i];
          bi[i] = take ? row : bi[i];
        }
      }
    } else {
      const int64_t left = N - r0;  // >= 1
      const bool writer = ks == 0 && j == 0;
#pragma unroll
      for (int i = 0; i < MX; ++i) {
        if (i > 0 && m + i >= M) continue;  // the missing second row (uniform)
        const __amdgpu_buffer_rsrc_t ys = __builtin_amdgcn_make_buffer_rsrc(
            Y + static_cast<int64_t>(m + i) * N + r0, 0,
            static_cast<int>((left < ROWS ? left : ROWS) * 4), 0x00020000);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float val = acc[i][r];
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), ys,
                                                writer ? (grp * R + r) * 4 : 0x40000000, 0, 0);
        }
      }
    }
  };

  // ping-pong over passes, two in flight; passes past the end read as zeros
  // (no traffic)
  for (;;) {
    float acc[MX][R];
    compute(wa, acc);
    finish(row0, acc, 0);
    const int64_t r1 = row0 + stride;
    if (r1 >= N) break;
    load(r1 + stride, wa);
    __builtin_amdgcn_sched_barrier(0);
    float acc2[MX][R];
    compute(wb, acc2);
    finish(r1, acc2, 1);
    row0 = r1 + stride;
    if (row0 >= N) break;
    load(row0 + stride, wb);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (ARGMAX) {
#pragma unroll
    for (int i = 0; i < MX; ++i) {
      if (i > 0) {
        if (m + i >= M) break;  // the missing second row (uniform)
        __syncthreads();        // the previous row's publish is done with its LDS
      }
      am_publish(bv[i], bi[i], m + i, workspace, static_cast<int>(gridDim.x), out_idx, out_val, W,
                 Y, N, K);
    }
  }
}

// Generic kernel: any K % 32 == 0 (odd block counts, very long rows).  16
// lanes per row, one block per lane per step, x read from global memory.
template <bool ARGMAX>
__global__ __launch_bounds__(256) void matvec_any_kernel(
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
        float s = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) s = nib_dot4_centred(qs[t], xb[t], xb[4 + t], s);
        acc = __builtin_fmaf(half_bits_to_float(d16), s, acc);
      }
    }
    const float v = row16_sum(acc);
    if constexpr (ARGMAX) {
      if (ok && am_better(v, static_cast<int>(row), bv, bi)) { bv = v; bi = static_cast<int>(row); }
    } else {
      if (ok && j == 0) Y[static_cast<int64_t>(m) * N + row] = v;
    }
  }
  if constexpr (ARGMAX)
    am_publish(bv, bi, m, workspace, static_cast<int>(gridDim.x), out_idx, out_val, W, Y, N, K);
}

// Grid of the pair kernel with R rows per lane: the fewest passes per
// workgroup that fit the resident workgroups, spread evenly (an uneven last
// round costs a whole pass).  A persistent grid must not exceed what is
// resident at once: a second, partial round of workgroups costs far more than
// it adds.
struct PairGrid {
  int64_t g;         // workgroups
  int64_t cu_rows;   // rows handled by the busiest CU
};
template <int KS, bool ARGMAX, int R, bool XL, int G, int MX = 1>
PairGrid pair_grid(int64_t N) {
  // per process (the kernel's resource use is fixed); racing first calls
  // store the same value
  static std::atomic<int> per_cu_cache{0};
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, matvec_pairs_kernel<KS, ARGMAX, R, XL, G, MX>,
                                                      64 * KS * G, 0) != hipSuccess || nb < 1)
      nb = 1;
    per_cu = nb;
    per_cu_cache.store(nb, std::memory_order_relaxed);
  }
  const int64_t cus = device_info().cu_count;
  const int64_t passes = (N + 4 * R * G - 1) / (4 * R * G);
  const int64_t cap = cus * per_cu;
  const int64_t rounds = (passes + cap - 1) / cap;
  const int64_t g = (passes + rounds - 1) / rounds;
  return PairGrid{g, ((g + cus - 1) / cus) * rounds * 4 * R * G};
}

// Rows up to 4096 long (KS <= 4), plain products: x in LDS, one row per lane
// and pass, 8 waves per SIMD -- measured 3-12 % faster than x in registers on
// the decoder shapes.  Tall matrices (the 131072-row LM head, as a matvec or
// with the argmax) take four row groups per workgroup sharing one copy of x
// in LDS: a quarter of the workgroups, each pass 16 contiguous rows (-4 % on
// both; slower on the decoder shapes, where each workgroup runs only a few
// passes).  Longer rows keep x in registers (each workgroup stages x once and
// runs few passes), and so does the argmax of shorter tables.  There, two
// rows per lane amortise the per-pass reductions and the per-workgroup
// start-up; one row per lane halves the pass granularity and is used only
// where two would leave CUs idle and one gives the busiest CU fewer rows.
constexpr int64_t MV_GROUPED_ROWS = 65536;
enum PairVariant { PV_LDS_G4, PV_LDS, PV_REG_R1, PV_REG_R2 };
template <int KS, bool ARGMAX>
PairVariant pair_variant(int64_t N) {
  if (KS <= 4 && N >= MV_GROUPED_ROWS) return PV_LDS_G4;
  if (KS <= 4 && !ARGMAX) return PV_LDS;
  const PairGrid g2 = pair_grid<KS, ARGMAX, 2, false, 1>(N);
  const PairGrid g1 = pair_grid<KS, ARGMAX, 1, false, 1>(N);
  const bool one = g2.g < device_info().cu_count && g1.g > g2.g && g1.cu_rows < g2.cu_rows;
  return one ? PV_REG_R1 : PV_REG_R2;
}

// Two or more rows of x are taken two per workgroup (the weights are read
// and decoded once per pair of rows), with x in registers at one weight row
// per lane (two rows of x at R = 2 would spill).  The argmax pairs rows only
// with x in LDS (the tall tables): with x in registers its second row's
// bookkeeping halves the occupancy.
template <int KS, bool ARGMAX, int R, bool XL, int G>
void launch_variant(const uint8_t* w, const float* x, float* y, int32_t* idx, float* val, void* ws,
                    int64_t M, int64_t N, int64_t K, hipStream_t s) {
  if constexpr (!ARGMAX || XL) {
    if (M >= 2) {
      constexpr int R2 = XL ? R : 1;
      const PairGrid g = pair_grid<KS, ARGMAX, R2, XL, G, 2>(N);
      hipLaunchKernelGGL((matvec_pairs_kernel<KS, ARGMAX, R2, XL, G, 2>),
                         dim3(static_cast<unsigned>(g.g), static_cast<unsigned>((M + 1) / 2)),
                         dim3(64 * KS * G), 0, s, w, x, y, idx, val, ws, N, static_cast<int>(K),
                         static_cast<int>(M));
      return;
    }
  }
  const PairGrid g = pair_grid<KS, ARGMAX, R, XL, G, 1>(N);
  hipLaunchKernelGGL((matvec_pairs_kernel<KS, ARGMAX, R, XL, G, 1>),
                     dim3(static_cast<unsigned>(g.g), M), dim3(64 * KS * G), 0, s, w, x, y, idx,
                     val, ws, N, static_cast<int>(K), static_cast<int>(M));
}

template <int KS, bool ARGMAX>
void launch_pairs(const uint8_t* w, const float* x, float* y, int32_t* idx, float* val, void* ws,
                  int64_t M, int64_t N, int64_t K, hipStream_t s) {
  switch (pair_variant<KS, ARGMAX>(N)) {
    case PV_LDS_G4:
      if constexpr (KS <= 4) launch_variant<KS, ARGMAX, 1, true, 4>(w, x, y, idx, val, ws, M, N, K, s);
      break;
    case PV_LDS:
      if constexpr (KS <= 4 && !ARGMAX)
        launch_variant<KS, ARGMAX, 1, true, 1>(w, x, y, idx, val, ws, M, N, K, s);
      break;
    case PV_REG_R1:
      launch_variant<KS, ARGMAX, 1, false, 1>(w, x, y, idx, val, ws, M, N, K, s);
      break;
    case PV_REG_R2:
      launch_variant<KS, ARGMAX, 2, false, 1>(w, x, y, idx, val, ws, M, N, K, s);
      break;
  }
}

// Pair-kernel waves per workgroup for K, or 0 for the generic kernel (K % 64
// == 32, or rows longer than 12288: more than 12 waves per workgroup would cap
// registers below the lane's x slice).
int64_t pair_ks(int64_t K) { return (K % 64 == 0 && K <= 12288) ? (K / 64 + 15) / 16 : 0; }

template <bool ARGMAX>
const char* route_mv(int64_t N, int64_t K) {
  static const char* names[] = {"pairs_lds_g4", "pairs_lds", "pairs_reg_r1", "pairs_reg_r2"};
  switch (pair_ks(K)) {
#define Q4_MV_CASE(n) \
  case n: return names[pair_variant<n, ARGMAX>(N)];
    Q4_MV_CASE(1) Q4_MV_CASE(2) Q4_MV_CASE(3) Q4_MV_CASE(4) Q4_MV_CASE(5) Q4_MV_CASE(6)
    Q4_MV_CASE(7) Q4_MV_CASE(8) Q4_MV_CASE(9) Q4_MV_CASE(10) Q4_MV_CASE(11) Q4_MV_CASE(12)
#undef Q4_MV_CASE
    default: return "any";
  }
}

template <bool ARGMAX>
hipError_t launch_mv(const uint8_t* w, const float* x, float* y, int32_t* idx, float* val,
                     void* ws, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  switch (pair_ks(K)) {
#define Q4_MV_CASE(n) \
  case n: launch_pairs<n, ARGMAX>(w, x, y, idx, val, ws, M, N, K, s); break;
    Q4_MV_CASE(1) Q4_MV_CASE(2) Q4_MV_CASE(3) Q4_MV_CASE(4) Q4_MV_CASE(5) Q4_MV_CASE(6)
    Q4_MV_CASE(7) Q4_MV_CASE(8) Q4_MV_CASE(9) Q4_MV_CASE(10) Q4_MV_CASE(11) Q4_MV_CASE(12)
#undef Q4_MV_CASE
    default: {
      const int cu = device_info().cu_count;
      int64_t g = (N + 15) / 16;
      const int64_t cap = static_cast<int64_t>(cu) * 8;
      if (g > cap) g = cap;
      hipLaunchKernelGGL((matvec_any_kernel<ARGMAX>), dim3(static_cast<unsigned>(g), M), dim3(256),
                         0, s, w, x, y, idx, val, ws, N, static_cast<int>(K));
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_matvec(const uint8_t* w, const float* x, float* y, int64_t M, int64_t N,
                         int64_t K, hipStream_t s) {
  return launch_mv<false>(w, x, y, nullptr, nullptr, nullptr, M, N, K, s);
}

const char* matvec_route(int64_t N, int64_t K, bool argmax) {
  return argmax ? route_mv<true>(N, K) : route_mv<false>(N, K);
}

size_t lmhead_workspace_bytes(int64_t M) {
  return static_cast<size_t>(M) * AM_ROW_BYTES;
}

hipError_t launch_lmhead_argmax(const uint8_t* w, const float* x, int32_t* out_idx, float* out_val,
                                float* out_embed, int64_t M, int64_t N, int64_t K, void* workspace,
                                hipStream_t s) {
  // in the argmax kernels the output pointer Y carries the embedding rows
  return launch_mv<true>(w, x, out_embed, out_idx, out_val, workspace, M, N, K, s);
}

// ---------------------------------------------------------------------------
// The argmax for callers that cannot allocate: its workspace (the per-row
// key and arrival counter, zero between calls) is this file-scope array,
// one copy per GPU, held until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device memory: the device address
// comes from hipGetSymbolAddress, taken once per device (with that device
// current) at the first call there, and only that address is passed on.
// The first call on a device also clears the array with a fill kernel on
// its stream; every completed call leaves it zero again.
// ---------------------------------------------------------------------------
constexpr int NOALLOC_MAX_M = 64;
static __device__ __align__(256) uint8_t scratch[NOALLOC_MAX_M * AM_ROW_BYTES];

__global__ void clear_words_kernel(uint32_t* p, int n) {
  const int i = static_cast<int>(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0u;
}

namespace {
constexpr int kNoallocDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoallocDevices];   // device address of `scratch`, per device
bool g_scratch_cleared[kNoallocDevices];
}  // namespace

int64_t lmhead_noalloc_max_m() { return NOALLOC_MAX_M; }

hipError_t launch_lmhead_argmax_noalloc(const uint8_t* w, const float* x, int32_t* out_idx,
                                        float* out_val, int64_t M, int64_t N, int64_t K,
                                        hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kNoallocDevices) return hipErrorInvalidDevice;
  void* ptr = nullptr;
  bool clear = false;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (ptr == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev] = ptr;
    }
    ptr = g_scratch_ptr[dev];
    clear = !g_scratch_cleared[dev];
    g_scratch_cleared[dev] = true;
  }
  if (clear) {
    const int words = NOALLOC_MAX_M * AM_ROW_BYTES / 4;
    hipLaunchKernelGGL(clear_words_kernel, dim3((words + 255) / 256), dim3(256), 0, s,
                       static_cast<uint32_t*>(ptr), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_mv<true>(w, x, nullptr, out_idx, out_val, ptr, M, N, K, s);
}

}  // namespace q4
