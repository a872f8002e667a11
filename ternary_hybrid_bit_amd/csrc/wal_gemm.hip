// Batched kernels of libwal for gfx950: Y = X W^T for bf16 activation rows on
// the 2-bit planes, from a few rows (multi-sequence decode) to prefill sizes.
// With B activation rows every decoded trit feeds B products:
//     Y[n][row] = sum_g ( alpha[row][g] * sum_{k in g} T[row][k] X[n][k]
//                       +  beta[row][g] * sum_{k in g} R[row][k] X[n][k] )
//               + sum_t (-1)^{U bit} z[n][t]
// (WAL-Ternary-8B cards, "Representation": the ternary-hybrid product and its
// binary low-rank paths; the per-(row, group) scales are applied in fp32).
//
// Batched GEMV (k_gemv_batch, vector ALUs, B <= 32), two launches:
//  1. a wavefront takes kGemvRows rows of one 4096-column pass for up to
//     kGemvCols columns and writes its partial sums P[pass][n][row].  Each
//     lane decodes its 64 trits of a row once (shift and mask to bf16 +-2 / 0,
//     as the batch-1 kernels do) and feeds them to one v_dot2_f32_bf16 per
//     trit pair and column; the sites gather 2x from a per-pass LDS copy of X.
//     Extra workgroups at the end of the grid write the low-rank reductions
//     of every batch column per 4096-column chunk, zpart[chunk][n][t];
//  2. k_reduce adds the passes and the chunks in a fixed order, adds the
//     low-rank term and stores Y.
// Matrix cores (k_mfma for B <= 32, k_prefill beyond): the trits of a 16-row
// tile become bf16 A operands of v_mfma_f32_16x16x32_bf16 (lane (row i =
// lane & 15, K block kb = lane >> 4) decodes its 8 code bytes with one 64-bit
// shift and a mask per operand pair); the group's sites are scattered as +-2
// into a per-wavefront LDS tile in operand order, read back as a second A
// operand and cleared; X is staged once per workgroup in LDS in operand order
// and read as the B operand.  The T and R group sums land in separate
// accumulators that alpha and beta scale in fp32.  k_mfma writes partial sums
// per 1024-column slice for k_reduce; k_prefill sweeps all columns (split
// along K only when its tiles would not fill the GPU) and writes Y with the
// low-rank term of k_zmma's partials.  Decoded values are exact in bf16 and
// every product and sum is fp32, so x = e_j still gives column j of W
// exactly, and every sum runs in a fixed order: results do not depend on
// timing.
#include <hip/hip_runtime.h>

#include "wal_device.h"
#include "wal_internal.h"

namespace {


template <int SF>
__device__ __forceinline__ float scale_value(uint32_t raw) {
  if constexpr (SF == WAL_SCALE_FP16) return (float)__builtin_bit_cast(_Float16, (uint16_t)raw);
  return __uint_as_float(raw << 8);
}

template <int K>
__device__ __forceinline__ uint32_t load_sites(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (K == 8) return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kStream);
  if constexpr (K == 4) return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kStream);
  return __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, kStream);
}

// Lane n of each row of 16 lanes, to the whole row (DPP row_newbcast).
__device__ __forceinline__ uint32_t row_bcast(uint32_t v, uint32_t n) {
  switch (n) {
#define WAL_BC(N) case N: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x150 + N, 0xF, 0xF, true);
    WAL_BC(0) WAL_BC(1) WAL_BC(2) WAL_BC(3) WAL_BC(4) WAL_BC(5) WAL_BC(6) WAL_BC(7)
    WAL_BC(8) WAL_BC(9) WAL_BC(10) WAL_BC(11) WAL_BC(12) WAL_BC(13) WAL_BC(14) default: WAL_BC(15)
#undef WAL_BC
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// Low-rank partials: block b of the z part of a grid computes, for batch
// column n, terms 16 tc .. 16 tc + 15 over columns [4096 cc, 4096 cc + 4096).
__device__ __forceinline__ void z_block(const MatDev& d, float* __restrict__ zpart, uint32_t b) {
  const uint32_t tcs = (d.terms + kZTermsPerBlock - 1) / kZTermsPerBlock;
  const uint32_t tc = b % tcs, rest = b / tcs, n = rest % d.batch, cc = rest / d.batch;
  const void* x = reinterpret_cast<const uint16_t*>(d.x) + (size_t)n * d.ldx;
  float* out = zpart + ((size_t)cc * d.batch + n) * d.terms;
  const uint32_t c0 = cc * kZChunkCols, c1 = min(d.in, c0 + kZChunkCols);
  z_chunk<WAL_X_BF16, (int)kZTermsPerBlock, kZOutDev>(d, x, tc * kZTermsPerBlock, out, c0, c1);
}

uint32_t z_blocks(const MatDev& d, const GemmShape& S) {
  return d.terms ? S.zc * d.batch * ((d.terms + kZTermsPerBlock - 1) / kZTermsPerBlock) : 0;
}

// Y[n][row] = sum over K slices of the partials (in slice order) + the
// low-rank term with z[n][t] = sum over chunks of zpart (in chunk order).
// Every load is issued before the first sum, so the kernel pays one memory
// latency, not one per slice, chunk or U byte.
constexpr uint32_t kReduceSlices = 16;  // partial slices loaded ahead (more: a loop)
constexpr uint32_t kReduceChunks = 8;   // z chunks loaded ahead

__global__ __launch_bounds__(256) void k_reduce(MatDev d, const float* __restrict__ zpart,
                                                const float* __restrict__ P, uint32_t slices, uint32_t zc) {
  __shared__ float zs[kMaxTerms];
  const uint32_t n = blockIdx.y, row = blockIdx.x * 256 + threadIdx.x;
  const uint32_t rr = min(row, d.out - 1);
  const size_t plane = (size_t)d.batch * d.out, at = (size_t)n * d.out + rr;
  float pv[kReduceSlices];
#pragma unroll
  for (uint32_t s = 0; s < kReduceSlices; ++s) pv[s] = s < slices ? P[s * plane + at] : 0.f;
  const uint32_t ub = (d.rank + 7) / 8;   // at most 8
  uint32_t ubyte[WAL_MAX_PATHS][8];
#pragma unroll
  for (uint32_t p = 0; p < WAL_MAX_PATHS; ++p)
#pragma unroll
    for (uint32_t j = 0; j < 8; ++j)
      ubyte[p][j] = p < d.n_paths && j < ub ? path_plane(d.U, d, p)[(size_t)rr * ub + j] : 0u;
  uint64_t ubits[WAL_MAX_PATHS];   // the row's U bits of path p, rank r at bit r
#pragma unroll
  for (uint32_t p = 0; p < WAL_MAX_PATHS; ++p) {
    ubits[p] = 0;
#pragma unroll
    for (uint32_t j = 0; j < 8; ++j) ubits[p] |= (uint64_t)ubyte[p][j] << (8 * j);
  }
  const uint32_t t = threadIdx.x;
  float zv[kReduceChunks];
#pragma unroll
  for (uint32_t cc = 0; cc < kReduceChunks; ++cc)
    zv[cc] = t < d.terms && cc < zc ? zpart[((size_t)cc * d.batch + n) * d.terms + t] : 0.f;
  if (t < d.terms) {
    float z = zv[0];
#pragma unroll
    for (uint32_t cc = 1; cc < kReduceChunks; ++cc) z += zv[cc];
    for (uint32_t cc = kReduceChunks; cc < zc; ++cc) z += zpart[((size_t)cc * d.batch + n) * d.terms + t];
    zs[t] = z;
  }
  __syncthreads();
  if (row >= d.out) return;
  float v = pv[0];
#pragma unroll
  for (uint32_t s = 1; s < kReduceSlices; ++s) v += pv[s];
  for (uint32_t s = kReduceSlices; s < slices; ++s) v += P[s * plane + at];
#pragma unroll
  for (uint32_t p = 0; p < WAL_MAX_PATHS; ++p) {
    if (p >= d.n_paths) break;
    for (uint32_t r = 0; r < d.rank; ++r) {
      const float zt = zs[p * d.rank + r];
      v += ((ubits[p] >> r) & 1u) ? -zt : zt;
    }
  }
  d.y[(size_t)n * d.ldy + row] = v;
}

// ---------------------------------------------------------------------------
// Batched GEMV.  Pairs of a lane: p[n][8 dw + i] = (X[n][c + 16 dw + i],
// X[n][c + 16 dw + 8 + i]), the columns whose codes sit at bits 2i and
// 2i + 16 of the lane's code dword dw.

template <int NB, int I>
__device__ __forceinline__ void dot_batch(uint64_t q, int h, const uint32_t (&p)[NB][32], float (&a)[NB]) {
  const uint64_t t = shl64<14 - 2 * I>(q);
  const uint32_t lo = (uint32_t)t & 0xC000C000u, hi = (uint32_t)(t >> 32) & 0xC000C000u;
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    a[n] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lo),
                                           __builtin_bit_cast(bf16x2_t, p[n][16 * h + I]), a[n], false);
    a[n] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, hi),
                                           __builtin_bit_cast(bf16x2_t, p[n][16 * h + 8 + I]), a[n], false);
  }
  if constexpr (I < 7) dot_batch<NB, I + 1>(q, h, p, a);
}

// Block b < nmain: pass b % passes, rows of block (b / passes) % nrb, batch
// columns NB * (b / (passes * nrb)) ..; blocks past nmain: low-rank partials.
template <int SF, int K, int NB>
__global__ __launch_bounds__(kThreads) void k_gemv_batch(MatDev d, float* __restrict__ P, float* __restrict__ zpart,
                                                         uint32_t nmain, uint32_t passes, uint32_t nrb) {
  if (blockIdx.x >= nmain) {
    z_block(d, zpart, blockIdx.x - nmain);
    return;
  }
  // X of the pass, doubled, as [column][NB] bf16: the site gathers
  __shared__ uint16_t tbl[kPass2bit * NB];
  constexpr uint32_t R = kGemvRows * NB;
  constexpr uint32_t SB = SF == WAL_SCALE_FP16 ? 2 : 3;
  const uint32_t pass = blockIdx.x % passes, rest = blockIdx.x / passes;
  const uint32_t c0 = (rest / nrb) * NB;
  const uint32_t row_base = (rest % nrb) * (kWaves * kGemvRows) + wave_id() * kGemvRows;
  const uint32_t col0 = pass * kPass2bit, pw = min(kPass2bit, d.in - col0);
  const int lane = threadIdx.x & 63;
  const bool active = (uint32_t)lane * 64 < pw;
  const uint16_t* X = reinterpret_cast<const uint16_t*>(d.x);

  // Weights first: every row of the wavefront (rows past the matrix repeat
  // its last row; lanes past the pass width read their row's last group, in
  // bounds, with zero x and scales).
  const uint32_t G = d.groups;
  const uint32_t g = min(pass * (kPass2bit / 128) + (lane >> 1), G - 1), h = lane & 1;
  const uint32_t cvoff = min(col0 / 4 + lane * 16, d.row_stride - 16);
  const __amdgpu_buffer_rsrc_t rc = rsrc(d.codes, d.blob_bytes);
  const __amdgpu_buffer_rsrc_t ra = rsrc(d.alpha, d.blob_bytes - (uint32_t)(d.alpha - d.codes));
  __amdgpu_buffer_rsrc_t rs = rsrc(d.codes, 0u), rb = rsrc(d.codes, 0u);
  if constexpr (K > 0) {
    rs = rsrc(d.sites, d.blob_bytes - (uint32_t)(d.sites - d.codes));
    rb = rsrc(d.beta, d.blob_bytes - (uint32_t)(d.beta - d.codes));
  }
  u32x4_t c[kGemvRows];
  uint32_t sa[kGemvRows], sbeta[kGemvRows], st[kGemvRows];
#pragma unroll
  for (uint32_t j = 0; j < kGemvRows; ++j) {
    const uint32_t row = min(row_base + j, d.out - 1);
    c[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rc, cvoff, row * d.row_stride,
                                                                             kStream));
    sa[j] = load_scale<SF>(ra, g * SB, row * G * SB);
    if constexpr (K > 0) {
      sbeta[j] = load_scale<SF>(rb, g * SB, row * G * SB);
      st[j] = load_sites<K>(rs, g * K + h * (K / 2), row * G * K);
    }
  }

  // x pairs of the lane's 64 columns, every batch column of the block
  uint32_t p[NB][32];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    if (active && c0 + n < d.batch) {
      const uint4* src = reinterpret_cast<const uint4*>(X + (size_t)(c0 + n) * d.ldx + col0 + lane * 64);
      uint32_t w[32];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint4 v = src[q];
        w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
      }
#pragma unroll
      for (int dw = 0; dw < 4; ++dw)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int lo = 16 * dw + i, hi = 16 * dw + 8 + i;
          p[n][8 * dw + i] = ((w[lo >> 1] >> (16 * (lo & 1))) & 0xFFFFu) |
                             (((w[hi >> 1] >> (16 * (hi & 1))) & 0xFFFFu) << 16);
        }
    } else {
#pragma unroll
      for (int q = 0; q < 32; ++q) p[n][q] = 0;
    }
  }
  // site table: 8 columns of one batch column per thread and step (a fixed
  // trip count, so every load is issued before the first store)
#pragma unroll
  for (uint32_t it = 0; it < kPass2bit / 8 * NB / kThreads; ++it) {
    const uint32_t e = threadIdx.x + it * kThreads;
    const uint32_t n = e % NB, c8 = (e / NB) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (c8 < pw && c0 + n < d.batch) v = *reinterpret_cast<const uint4*>(X + (size_t)(c0 + n) * d.ldx + col0 + c8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t b = (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
      tbl[(c8 + k) * NB + n] = (uint16_t)(__float_as_uint(2.0f * __uint_as_float(b << 16)) >> 16);
    }
  }
  __syncthreads();

  float acc[R];
#pragma unroll
  for (uint32_t j = 0; j < kGemvRows; ++j) {
    float t[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) t[n] = 0.f;
    dot_batch<NB, 0>(((uint64_t)c[j][1] << 32) | c[j][0], 0, p, t);
    dot_batch<NB, 0>(((uint64_t)c[j][3] << 32) | c[j][2], 1, p, t);
    const float al = active ? scale_value<SF>(sa[j]) : 0.f;
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[j * NB + n] = al * t[n];
    if constexpr (K > 0) {
      float r[NB];
#pragma unroll
      for (int n = 0; n < NB; ++n) r[n] = 0.f;
#pragma unroll
      for (int q = 0; q < K / 2; ++q) {
        const uint32_t sb = (st[j] >> (8 * q)) & 0xFFu;
        const uint32_t idx = (lane >> 1) * 128 + (sb & 127u);
        const uint32_t flip = (0u - (sb >> 7)) & 0x80008000u;
        if constexpr (NB == 4) {
          const uint2 v = *reinterpret_cast<const uint2*>(&tbl[idx * 4]);
          const uint32_t v0 = v.x ^ flip, v1 = v.y ^ flip;
          r[0] += bf16_lo(v0); r[1] += bf16_hi(v0); r[2] += bf16_lo(v1); r[3] += bf16_hi(v1);
        } else if constexpr (NB == 2) {
          const uint32_t v = *reinterpret_cast<const uint32_t*>(&tbl[idx * 2]) ^ flip;
          r[0] += bf16_lo(v); r[1] += bf16_hi(v);
        } else {
          r[0] += bf16_lo((uint32_t)tbl[idx] ^ flip);
        }
      }
      const float be = active ? scale_value<SF>(sbeta[j]) : 0.f;
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[j * NB + n] = __builtin_fmaf(be, r[n], acc[j * NB + n]);
    }
  }
  const float tot = treduce<R>(acc, lane);
  constexpr int SH = 6 - ilog2(R);
  if ((lane & ((1 << SH) - 1)) == 0) {
    const uint32_t v = lane >> SH, j = v / NB, n = c0 + v % NB, row = row_base + j;
    if (row < d.out && n < d.batch) P[((size_t)pass * d.batch + n) * d.out + row] = 0.5f * tot;
  }
}

// ---------------------------------------------------------------------------
// MFMA path.

__device__ __forceinline__ f32x4_t mfma(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// B operands of one group for one n-tile: lane (n, kb) holds X[n][128 g + 32 kb
// + c], c < 32, as w[16] (bf16 pairs in memory order); operand m, pair q is
// (X[.][K_lo], X[.][K_lo + 8]) with o = 4m + q, K_lo = 16 (o >> 3) + (o & 7):
// the trit pair the A-operand decode puts in the same slot.
__device__ __forceinline__ void x_operands(const uint4 (&raw)[4], uint4 (&b)[4]) {
  const uint32_t w[16] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w,
                          raw[2].x, raw[2].y, raw[2].z, raw[2].w, raw[3].x, raw[3].y, raw[3].z, raw[3].w};
  uint32_t o4[16];
#pragma unroll
  for (int o = 0; o < 16; ++o) {
    const int lo = 16 * (o >> 3) + (o & 7);   // hi = lo + 8: same half of w[lo / 2 + 4]
    // one v_perm_b32: low or high halves of the two dwords
    o4[o] = __builtin_amdgcn_perm(w[(lo >> 1) + 4], w[lo >> 1], (lo & 1) ? 0x07060302u : 0x05040100u);
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) b[m] = make_uint4(o4[4 * m], o4[4 * m + 1], o4[4 * m + 2], o4[4 * m + 3]);
}

// T operands of one group from the lane's 8 code bytes (q: dword 1 : dword
// 0): operand m, pair k holds the trits of columns 16 (o >> 3) + (o & 7) and
// + 8, o = 4m + k, as bf16 +-2 / 0.  A 64-bit shift positions the pairs of
// both dwords at once (pairs o and o + 8 share a shift).
template <int I>
__device__ __forceinline__ void a_operands(uint64_t q, uint4 (&a)[4]) {
  const uint64_t s = shl64<14 - 2 * I>(q);
  const uint32_t lo = (uint32_t)s & 0xC000C000u, hi = (uint32_t)(s >> 32) & 0xC000C000u;
  // o = I (dword 0) and o = 8 + I (dword 1)
  reinterpret_cast<uint32_t*>(&a[I >> 2])[I & 3] = lo;
  reinterpret_cast<uint32_t*>(&a[2 + (I >> 2)])[I & 3] = hi;
  if constexpr (I < 7) a_operands<I + 1>(q, a);
}

// MFMA kernels' work split: a workgroup of kMfmaTiles wavefronts takes
// kMfmaTiles 16-row tiles (one per wavefront) and sweeps its columns kSlots
// 128-column groups at a time.  Every wavefront needs the same X for a sweep,
// so the workgroup stages it once in LDS and each wavefront reads its B
// operands from there: X crosses from L2 once per kMfmaTiles tiles instead of
// once per tile.  k_mfma (small batch) gives a workgroup one kSliceCols-column
// slice (kSweeps sweeps) and writes partial sums; k_prefill (large batch)
// gives it every column of a 32-row batch chunk and writes Y.
// Four tiles per workgroup (measured on the 4096 x 12288 shape, us per call
// at batch 1 / 8 / 32): 16.2 / 17.0 / 24.4, against 17.9 / 19.1 / 25.8 with
// eight and 17.6 / 20.0 / 32.6 with two; 512- or 2048-column slices were
// slower with either.
constexpr uint32_t kSlots = 4;
constexpr uint32_t kSweeps = kSliceCols / 128 / kSlots;
constexpr uint32_t kMfmaTiles = 4;
constexpr uint32_t kMfmaWaves = kMfmaTiles;

// X rows nbase .. nbase + 16 NT - 1 of one sweep of SL groups in LDS, in
// MFMA operand order: one 1 KB block per (n-tile t, slot q, operand m) in
// which lane L = (n, kb) finds its B operand at 16 L, so that every
// B-operand read of a wavefront is one contiguous 1 KB (the only ds_read_b128
// pattern free of bank conflicts on gfx950; row-padded layouts are not).
// Operand m of lane (n, kb) holds the pairs (column k, column k + 8), k =
// 4 (m & 1) .. + 3, of the 16-column half m >> 1 of the lane's 32-column block
// kb: the trit pairs that the A-operand decode puts in the same slots.
// Staging job j (one wavefront instruction pair) covers (t, q, half h): lane L
// loads the 32 bytes of its row and half, permutes them into pair order and
// writes both 16-byte operand chunks at 16 L of blocks m = 2h and 2h + 1.
// The W wavefronts take the 2 NT SL jobs in turn.
template <int NT, int SL>
__device__ __forceinline__ uint32_t x_block(int t, uint32_t q, int m) { return ((t * SL + q) * 4 + m) * 1024; }

template <int NT, int W, int SL>
struct XStage {
  static constexpr uint32_t kBytes = NT * SL * 4 * 1024;
  static constexpr int kPer = 2 * NT * SL / W;  // jobs per wavefront
  static_assert(kPer * W == 2 * NT * SL, "whole jobs per wavefront");
  u32x4_t v[kPer][2];

  // X[n][128 (c0 + q) + 32 kb + 16 h .. + 16] of job j = wave + W u, zero
  // past the row's end (bit 31 set: X is smaller than 2 GiB, so the buffer
  // load returns zeros; an OR rather than a select keeps the address
  // arithmetic unconditional, so no branch splits the loop); rows past the
  // batch read row 0 (such B-operand columns only feed unused outputs).
  __device__ __forceinline__ void load(const MatDev& d, __amdgpu_buffer_rsrc_t rx, uint32_t c0, uint32_t nbase) {
    const uint32_t lane = threadIdx.x & 63, wave = wave_id();
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t j = wave + W * u, t = j / (2 * SL), q = (j / 2) % SL, h = j & 1;
      const uint32_t n = nbase + 16 * t + (lane & 15);
      const uint32_t col = 128 * (c0 + q) + 32 * (lane >> 4) + 16 * h;
      const uint32_t off = (2 * ((n < d.batch ? n : 0u) * d.ldx + col)) | (col < d.in ? 0u : 0x80000000u);
      v[u][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
      v[u][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16, 0, 0);
    }
  }

  // Pair dword k = (column k, column k + 8): low halves of dwords k / 2 and
  // k / 2 + 4 for even k, high halves for odd k (one v_perm_b32 each).
  __device__ __forceinline__ void store(uint8_t* xs) const {
    const uint32_t lane = threadIdx.x & 63, wave = wave_id();
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t j = wave + W * u, t = j / (2 * SL), q = (j / 2) % SL, h = j & 1;
      const uint32_t w[8] = {v[u][0][0], v[u][0][1], v[u][0][2], v[u][0][3],
                             v[u][1][0], v[u][1][1], v[u][1][2], v[u][1][3]};
      u32x4_t o[2];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        o[k >> 2][k & 3] = __builtin_amdgcn_perm(w[(k >> 1) + 4], w[k >> 1], (k & 1) ? 0x07060302u : 0x05040100u);
      *reinterpret_cast<u32x4_t*>(xs + x_block<NT, SL>(t, q, 2 * h) + 16 * lane) = o[0];
      *reinterpret_cast<u32x4_t*>(xs + x_block<NT, SL>(t, q, 2 * h + 1) + 16 * lane) = o[1];
    }
  }
};

// One wavefront's weights for one sweep of SL groups: lane (i, kb) holds the
// codes of row i of its tile (8 bytes per slot), its site bytes, and the
// scales of tile row 4 kb + (i & 3) for slot i >> 2 (so that each row of 16
// lanes holds the 4 x SL scales its C entries need, C holding rows 4 kb ..
// 4 kb + 3; a DPP row broadcast hands them out).
// Every field holds a load's result as loaded (16-bit or byte loads keep
// their own type): conversions happen where the values are used, so that no
// instruction needs a load before its sweep (a zero-extension hoisted to the
// loop head would wait for the next sweep's loads).
template <int SL>
struct SweepW {
  static_assert(SL == 2 || SL == 4, "sweeps of 2 or 4 groups");
  u32x4_t cw[SL / 2];      // codes of slots 2h, 2h + 1 (8 bytes each)
  uint16_t sites[SL];      // site byte(s) of the lane (K = 8: two, else one)
  uint16_t a16, b16;       // fp16 scales
  uint8_t a24[3], b24[3];  // fp24 scales, byte by byte
};

// Resources and fixed offsets of the weight loads.
struct WRes {
  __amdgpu_buffer_rsrc_t rc, ra, rs;
  uint32_t boff;   // beta plane from the alpha plane
};

template <int K>
__device__ __forceinline__ WRes make_wres(const MatDev& d) {
  WRes w;
  w.rc = rsrc(d.codes, d.blob_bytes);
  // one resource over the alpha and beta planes (beta at a fixed offset)
  w.ra = rsrc(d.alpha, d.blob_bytes - (uint32_t)(d.alpha - d.codes));
  w.boff = K > 0 ? (uint32_t)(d.beta - d.alpha) : 0u;
  w.rs = rsrc(d.codes, 0u);
  if constexpr (K > 0) w.rs = rsrc(d.sites, d.blob_bytes - (uint32_t)(d.sites - d.codes));
  return w;
}

// Groups c0 .. c0 + SL - 1 of the tile rows row_base .. + 15; groups at or
// past gend get zero scales (their codes and sites repeat the matrix's last
// group: in bounds, dropped by the zero scale).  The loads read 8 to 32
// bytes per row and instruction; the rest of each cache line is read
// moments later by the next slots, so they keep the default cache policy.
// K = 2: lanes kb and kb + 2 read the same site (their writes coincide).
template <int SF, int K, int SL>
__device__ __forceinline__ SweepW<SL> load_sweep(const MatDev& d, const WRes& w, uint32_t row_base, uint32_t c0,
                                                 uint32_t gend, int lane) {
  constexpr uint32_t SB = SF == WAL_SCALE_FP16 ? 2 : 3;
  const uint32_t i = lane & 15, kb = lane >> 4, G = d.groups;
  const uint32_t row = min(row_base + i, d.out - 1);
  SweepW<SL> s;
  {
    const uint32_t ra_row = min(row_base + 4 * kb + (i & 3), d.out - 1);
    const uint32_t g = c0 + (i >> 2);
    const uint32_t so = g < gend && (i >> 2) < (uint32_t)SL ? (ra_row * G + g) * SB : 0x7FFFFFF0u;
    if constexpr (SF == WAL_SCALE_FP16) {
      s.a16 = __builtin_amdgcn_raw_buffer_load_b16(w.ra, so, 0, 0);
      s.b16 = K > 0 ? __builtin_amdgcn_raw_buffer_load_b16(w.ra, so + w.boff, 0, 0) : (uint16_t)0;
    } else {
#pragma unroll
      for (int b = 0; b < 3; ++b) {
        s.a24[b] = __builtin_amdgcn_raw_buffer_load_b8(w.ra, so + b, 0, 0);
        s.b24[b] = K > 0 ? __builtin_amdgcn_raw_buffer_load_b8(w.ra, so + w.boff + b, 0, 0) : (uint8_t)0;
      }
    }
  }
#pragma unroll
  for (uint32_t q = 0; q < (uint32_t)SL; ++q) {
    const uint32_t g = min(c0 + q, G - 1);
    const u32x2_t c2 =
        __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(w.rc, row * d.row_stride + g * 32 + 8 * kb, 0, 0));
    s.cw[q / 2][2 * (q & 1)] = c2[0];
    s.cw[q / 2][2 * (q & 1) + 1] = c2[1];
    s.sites[q] = 0;
    if constexpr (K == 8) s.sites[q] = __builtin_amdgcn_raw_buffer_load_b16(w.rs, (row * G + g) * 8 + 2 * kb, 0, 0);
    if constexpr (K == 4) s.sites[q] = __builtin_amdgcn_raw_buffer_load_b8(w.rs, (row * G + g) * 4 + kb, 0, 0);
    if constexpr (K == 2) s.sites[q] = __builtin_amdgcn_raw_buffer_load_b8(w.rs, (row * G + g) * 2 + (kb & 1), 0, 0);
  }
  return s;
}

// The lane's raw alpha and beta bits (32-bit) of a loaded sweep.  The empty
// asm statements pin the conversion to the point of use: without them the
// compiler merges the fp24 bytes (and zero-extends fp16) where the loop-carried
// values meet, at the loop head, which then waits for loads still in flight.
__device__ __forceinline__ uint32_t pin(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}
template <int SF, int SL>
__device__ __forceinline__ uint32_t alpha_raw(const SweepW<SL>& w) {
  if constexpr (SF == WAL_SCALE_FP16) return pin(w.a16);
  return pin(w.a24[0]) | (pin(w.a24[1]) << 8) | (pin(w.a24[2]) << 16);
}
template <int SF, int SL>
__device__ __forceinline__ uint32_t beta_raw(const SweepW<SL>& w) {
  if constexpr (SF == WAL_SCALE_FP16) return pin(w.b16);
  return pin(w.b24[0]) | (pin(w.b24[1]) << 8) | (pin(w.b24[2]) << 16);
}

// The SL slots of a sweep for one wavefront and RT row tiles:
// C[r][t][j] += alpha sT + beta sR for row 4 kb + j of tile r and batch
// column 16 t + i (decoded values are 2x).  xs: the sweep's X in LDS
// (operand order); rtile: the wavefront's RT R tiles of 4 KB (zero on entry
// and on exit).  Each B operand read from LDS feeds the T and R products of
// all RT tiles: LDS bandwidth (about 128 bytes per clock and CU) is what
// bounds these kernels, and a 1 KB operand read per two MFMAs would use all
// of it.
template <int SF, int K, int NT, int RT, int SL>
__device__ __forceinline__ void sweep_mfma(const uint8_t* xs, const SweepW<SL> (&w)[RT], int lane, uint8_t* rtile,
                                           f32x4_t (&C)[RT][NT]) {
  const uint32_t i = lane & 15, kb = lane >> 4;
#pragma unroll
  for (uint32_t q = 0; q < (uint32_t)SL; ++q) {
    constexpr int PER = K == 8 ? 2 : 1;
    uint32_t addr[RT][PER];
    uint4 ro[RT][4];
    if constexpr (K > 0) {
      // lane (i, kb) scatters sites kb * K / 4 .. of row i (K = 2: site kb & 1,
      // lanes kb and kb + 2 writing the same value) into its R tiles, operand
      // m of lane L at [m][L]
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        uint16_t* rt16 = reinterpret_cast<uint16_t*>(rtile + 4096 * r);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const uint32_t sb = ((uint32_t)w[r].sites[q] >> (8 * j)) & 0xFFu;
          const uint32_t pos = sb & 127u, local = pos & 31u, rr = local & 15u;
          const uint32_t o = 8 * (local >> 4) + (rr & 7u);
          const uint32_t lt = (pos >> 5) * 16 + i;   // lane whose operand holds column pos of row i
          addr[r][j] = ((o >> 2) * 64 + lt) * 8 + (o & 3) * 2 + (rr >> 3);
          rt16[addr[r][j]] = (sb & 128u) ? 0xC000u : 0x4000u;
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int m = 0; m < 4; ++m) ro[r][m] = reinterpret_cast<const uint4*>(rtile + 4096 * r)[m * 64 + lane];
      wave_lds_sync();
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        uint16_t* rt16 = reinterpret_cast<uint16_t*>(rtile + 4096 * r);
#pragma unroll
        for (int j = 0; j < PER; ++j) rt16[addr[r][j]] = 0;
      }
    }
    // T operands: one 64-bit shift positions the code pairs of both dwords
    uint4 a[RT][4];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const uint64_t cq = ((uint64_t)w[r].cw[q / 2][2 * (q & 1) + 1] << 32) | w[r].cw[q / 2][2 * (q & 1)];
      a_operands<0>(cq, a[r]);
    }
    // scales of the lane's C rows 4 kb + j (a DPP row broadcast)
    float al[RT][4], be[RT][4];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const uint32_t araw = alpha_raw<SF>(w[r]), braw = K > 0 ? beta_raw<SF>(w[r]) : 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        al[r][j] = scale_value<SF>(row_bcast(araw, 4 * q + j));
        be[r][j] = K > 0 ? scale_value<SF>(row_bcast(braw, 4 * q + j)) : 0.f;
      }
    }
    // B operands of lane (n, kb) for X row 16 t + n: contiguous 1 KB reads,
    // those of n-tile t + 1 issued before the products of n-tile t (the
    // scheduling barriers keep the compiler from hoisting more of them)
    uint4 xn[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) xn[m] = *reinterpret_cast<const uint4*>(xs + x_block<NT, SL>(0, q, m) + 16 * lane);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint4 xb[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) xb[m] = xn[m];
      if (t + 1 < NT) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
          xn[m] = *reinterpret_cast<const uint4*>(xs + x_block<NT, SL>(t + 1, q, m) + 16 * lane);
      }
      f32x4_t sT[RT], sR[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        sT[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        sR[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          sT[r] = mfma(a[r][m], xb[m], sT[r]);
          if constexpr (K > 0) sR[r] = mfma(ro[r][m], xb[m], sR[r]);
        }
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          C[r][t][j] = __builtin_fmaf(al[r][j], sT[r][j], C[r][t][j]);
          if constexpr (K > 0) C[r][t][j] = __builtin_fmaf(be[r][j], sR[r][j], C[r][t][j]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The first nz blocks compute the low-rank partials (z_block), so that they
// run alongside the rest.  Block nz + b: row block b / slices (kMfmaTiles
// tiles, tile w to wavefront w) over column slice b % slices.  Wavefront w
// writes P[slice][n][row] = 0.5 sum over the slice's groups (alpha sT + beta
// sR) for its tile (decoded values are 2x).
template <int SF, int K, int NT>
__global__ __launch_bounds__(kMfmaWaves * 64) void k_mfma(MatDev d, float* __restrict__ P, float* __restrict__ zpart,
                                                           uint32_t nz, uint32_t slices) {
  if (blockIdx.x < nz) {
    z_block(d, zpart, blockIdx.x);
    return;
  }
  __shared__ __align__(16) uint8_t xs[XStage<NT, kMfmaWaves, kSlots>::kBytes];
  __shared__ __align__(16) uint8_t rts[kMfmaWaves * 4096];   // per-wavefront R tiles
  const int lane = threadIdx.x & 63;
  const uint32_t wave = wave_id();
  const uint32_t rb = (blockIdx.x - nz) / slices, slice = (blockIdx.x - nz) % slices;
  const uint32_t row_base = (rb * kMfmaTiles + wave) * 16;
  const uint32_t gs0 = slice * (kSliceCols / 128), gs1 = min(d.groups, gs0 + kSliceCols / 128);
  uint8_t* rtile = rts + wave * 4096;
  const WRes wr = make_wres<K>(d);
  const __amdgpu_buffer_rsrc_t rx = rsrc(d.x, 2 * ((d.batch - 1) * d.ldx + d.in));

  f32x4_t C[1][NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) C[0][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (K > 0) {
#pragma unroll
    for (int m = 0; m < 4; ++m) reinterpret_cast<uint4*>(rtile)[m * 64 + lane] = make_uint4(0, 0, 0, 0);
    wave_lds_sync();
  }

  // Every load of the slice first: X of both sweeps (L2), then the weights
  // of both sweeps (HBM).  Rows differ across the lanes, so the row offsets
  // go in the voffset.
  XStage<NT, kMfmaWaves, kSlots> xg[kSweeps];
#pragma unroll
  for (uint32_t sw = 0; sw < kSweeps; ++sw) xg[sw].load(d, rx, gs0 + sw * kSlots, 0);
  SweepW<kSlots> ws[kSweeps][1];
#pragma unroll
  for (uint32_t sw = 0; sw < kSweeps; ++sw) ws[sw][0] = load_sweep<SF, K, kSlots>(d, wr, row_base, gs0 + sw * kSlots, gs1, lane);
#pragma unroll
  for (uint32_t sw = 0; sw < kSweeps; ++sw) {
    if (gs0 + sw * kSlots >= gs1) break;   // block-uniform
    __syncthreads();   // the previous sweep's readers are done
    xg[sw].store(xs);
    __syncthreads();
    sweep_mfma<SF, K, NT, 1, kSlots>(xs, ws[sw], lane, rtile, C);
  }

  // the wavefront's tile: rows 4 kb + j, batch columns 16 t + i
  const uint32_t i = lane & 15, kb = lane >> 4;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t yr = row_base + 4 * kb + j, n = 16 * t + i;
      if (yr < d.out && n < d.batch) P[((size_t)slice * d.batch + n) * d.out + yr] = 0.5f * C[0][t][j];
    }
}

// Large batches (k_prefill): a workgroup of kPrefillWaves wavefronts takes
// prefill_rows(SF) rows (RT 16-row tiles per wavefront) by one
// kPrefillCols-row batch chunk (four n-tiles) over one range of sweeps: each
// decoded A operand feeds four n-tiles, and each B operand read from LDS the
// T and R products of the wavefront's row tiles.  A tile id t names (row block, chunk,
// K split); the ids run chunk group by chunk group (cgw chunks each), row
// block by row block within a group, so that tiles that run at the same time
// share their X chunks and weight rows.  The hardware hands consecutive
// workgroups to the 8 XCDs in turn, so block b takes id (b % 8) * per_xcd +
// b / 8: each XCD walks its own contiguous run of ids, and its L2 serves the
// reuse.  If nsplit == 1 the workgroup writes Y (with the low-rank term from
// the z partials [zc][batch][terms]), else its split's partial sums
// P[split][n][row] for k_reduce.
constexpr int kPrefillSL = (int)kPrefillSweepGroups;

template <int SF, int K>
__global__ __launch_bounds__(kPrefillWaves * 64) void k_prefill(MatDev d, PrefillShape pg,
                                                                 const float* __restrict__ zpart, uint32_t zc,
                                                                 float* __restrict__ P) {
  constexpr int NT = kPrefillCols / 16, W = kPrefillWaves, SL = kPrefillSL;
  constexpr int RT = SF == WAL_SCALE_FP16 ? 2 : 1;   // row tiles per wavefront
  static_assert(W * RT * 16 == prefill_rows(SF), "rows of a prefill workgroup");
  using XS = XStage<NT, W, SL>;
  __shared__ __align__(16) uint8_t xs[2][XS::kBytes];   // double-buffered sweeps; z in the epilogue
  __shared__ __align__(16) uint8_t rts[W * RT * 4096];   // R tiles
  static_assert(2 * XS::kBytes >= NT * 16 * kMaxTerms * 4, "z of a chunk fits the X buffers' space");
  const int lane = threadIdx.x & 63;
  const uint32_t wave = wave_id();
  const uint32_t t = (blockIdx.x % 8) * pg.per_xcd + blockIdx.x / 8;
  if (t >= pg.tiles) return;   // block-uniform
  const uint32_t per_group = pg.rblocks * pg.nsplit * pg.cgw;
  const uint32_t cg = t / per_group, rem0 = t % per_group;
  const uint32_t rb = rem0 / (pg.nsplit * pg.cgw), r2 = rem0 % (pg.nsplit * pg.cgw);
  const uint32_t split = r2 / pg.cgw, chunk = cg * pg.cgw + r2 % pg.cgw;
  if (chunk >= pg.chunks) return;   // block-uniform: the last group may be narrower
  const uint32_t row_base = rb * prefill_rows(SF) + wave * 16 * RT, nbase = chunk * kPrefillCols;
  // sweeps of this split: an even share, the first ones one longer
  const uint32_t q0 = pg.sweeps / pg.nsplit, rem = pg.sweeps % pg.nsplit;
  const uint32_t sw0 = split * q0 + min(split, rem), sw1 = sw0 + q0 + (split < rem ? 1u : 0u);
  const uint32_t G = d.groups, g0 = sw0 * SL, g1 = min(G, sw1 * SL);
  const uint32_t nsw = (g1 - g0 + SL - 1) / SL;   // >= 1
  uint8_t* rtile = rts + wave * RT * 4096;
  const WRes wr = make_wres<K>(d);
  const __amdgpu_buffer_rsrc_t rx = rsrc(d.x, 2 * ((d.batch - 1) * d.ldx + d.in));

  f32x4_t C[RT][NT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int u = 0; u < NT; ++u) C[r][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (K > 0) {
#pragma unroll
    for (int m = 0; m < 4 * RT; ++m) reinterpret_cast<uint4*>(rtile)[m * 64 + lane] = make_uint4(0, 0, 0, 0);
    wave_lds_sync();
  }

  // Sweep s computes from xs[s & 1] while the X of sweep s + 1 (loaded during
  // sweep s - 1) goes to the other buffer and the loads of sweep s + 2 are
  // issued; one barrier per sweep.  The loop runs two sweeps per trip, so
  // that the weights of even and odd sweeps keep registers of their own (no
  // copy waits for loads in flight), and always both: an odd count ends
  // with one sweep past the split, whose scales load as zero (it adds
  // exactly 0).  With no exit in the middle of a trip the loop entry and the
  // back edge leave the same loads in flight, so each sweep waits only for
  // its own data.  Loads past the split's last group read zero scales and X
  // (or in-bounds codes, sites and X that the zero scales drop).
  // (The scheduling barriers keep the prologue's loads in this order, the
  // order of the loop's back edge.)
  XS xg;
  SweepW<SL> wa[RT], wb[RT];
  xg.load(d, rx, g0, nbase);
#pragma unroll
  for (int r = 0; r < RT; ++r) wa[r] = load_sweep<SF, K, SL>(d, wr, row_base + 16 * r, g0, g1, lane);
  __builtin_amdgcn_sched_barrier(0);
  xg.store(xs[0]);
  __builtin_amdgcn_sched_barrier(0);
  xg.load(d, rx, g0 + SL, nbase);
#pragma unroll
  for (int r = 0; r < RT; ++r) wb[r] = load_sweep<SF, K, SL>(d, wr, row_base + 16 * r, g0 + SL, g1, lane);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  for (uint32_t sw = 0; sw < nsw; sw += 2) {   // block-uniform
    // (scheduling barriers: no work of one sweep moves into the other, where
    // it would wait for loads still in flight)
    __builtin_amdgcn_sched_barrier(0);
    sweep_mfma<SF, K, NT, RT, SL>(xs[0], wa, lane, rtile, C);
    xg.store(xs[1]);   // its last readers finished before the previous barrier
    {
      const uint32_t c2 = g0 + (sw + 2) * SL;
      xg.load(d, rx, c2, nbase);
#pragma unroll
      for (int r = 0; r < RT; ++r) wa[r] = load_sweep<SF, K, SL>(d, wr, row_base + 16 * r, c2, g1, lane);
    }
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    sweep_mfma<SF, K, NT, RT, SL>(xs[1], wb, lane, rtile, C);
    xg.store(xs[0]);
    {
      const uint32_t c3 = g0 + (sw + 3) * SL;
      xg.load(d, rx, c3, nbase);
#pragma unroll
      for (int r = 0; r < RT; ++r) wb[r] = load_sweep<SF, K, SL>(d, wr, row_base + 16 * r, c3, g1, lane);
    }
    __syncthreads();
  }

  const uint32_t i = lane & 15, kb = lane >> 4;
  if (pg.nsplit > 1) {   // block-uniform
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t yr = row_base + 16 * r + 4 * kb + j, n = nbase + 16 * u + i;
          if (yr < d.out && n < d.batch) P[((size_t)split * d.batch + n) * d.out + yr] = 0.5f * C[r][u][j];
        }
    return;
  }

  // z of the chunk's batch rows, summed over the column chunks in order,
  // into the X buffers' space (the loop ended with a barrier: no reader left)
  float* zs = reinterpret_cast<float*>(&xs[0][0]);   // [kPrefillCols][terms]
  for (uint32_t e = threadIdx.x; e < kPrefillCols * d.terms; e += blockDim.x) {
    const uint32_t n = nbase + e / d.terms, tt = e % d.terms;
    float z = 0.f;
    if (n < d.batch)
      for (uint32_t cc = 0; cc < zc; ++cc) z += zpart[((size_t)cc * d.batch + n) * d.terms + tt];
    zs[e] = z;
  }
  __syncthreads();
  // the wavefront's tiles: rows 16 r + 4 kb + j, batch columns nbase + 16 u
  // + i, plus sum_t (-1)^{U bit} z[n][t]
  const uint32_t ub = (d.rank + 7) / 8;
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t yr = row_base + 16 * r + 4 * kb + j;
      if (yr >= d.out) continue;
      float lr[NT] = {};
      for (uint32_t p = 0; p < d.n_paths; ++p) {
        const uint8_t* u8 = path_plane(d.U, d, p) + (size_t)yr * ub;
        for (uint32_t rr = 0; rr < d.rank; ++rr) {
          const bool neg = (u8[rr >> 3] >> (rr & 7)) & 1u;
#pragma unroll
          for (int u = 0; u < NT; ++u) {
            const float zt = zs[(16 * u + i) * d.terms + p * d.rank + rr];
            lr[u] += neg ? -zt : zt;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const uint32_t n = nbase + 16 * u + i;
        if (n < d.batch) d.y[(size_t)n * d.ldy + yr] = 0.5f * C[r][u][j] + lr[u];
      }
    }
}

// Low-rank reductions for k_prefill on the matrix cores:
//     zpart[ks][n][t] = s_t * sum over split ks's columns of (-1)^{V bit} X[n][c]
// (WAL-Ternary-8B cards, "Representation": the binary paths' V^T x).  One
// wavefront per (16 batch rows, 16 terms, column split): X is the A operand
// as stored (lane (n, kb) takes 8 consecutive columns, 16 bytes), and the
// lane (t, kb) of the B operand expands the matching 8 V bits of term t into
// +-1 bf16 (one V dword serves the four MFMAs of a 128-column group).  Rows
// past the batch read its last row and terms past the last term the last
// term's plane; neither is stored.
__global__ __launch_bounds__(64) void k_zmma(MatDev d, float* __restrict__ zpart, uint32_t groups_per_split) {
  const uint32_t lane = threadIdx.x, i = lane & 15, kb = lane >> 4;
  const uint32_t T = d.terms, ks = blockIdx.z;
  const uint32_t n = min(blockIdx.x * 16 + i, d.batch - 1);
  const uint32_t t = min(blockIdx.y * 16 + i, T - 1), p = t / d.rank, q = t % d.rank;
  const uint32_t g0 = ks * groups_per_split, g1 = min(d.groups, g0 + groups_per_split);
  const __amdgpu_buffer_rsrc_t rx = rsrc(d.x, 2 * ((d.batch - 1) * d.ldx + d.in));
  const __amdgpu_buffer_rsrc_t rv = rsrc(d.V, d.blob_bytes - (uint32_t)(d.V - d.codes));
  const uint32_t xoff = 2 * (n * d.ldx + 32 * kb), voff = p * d.pstride + q * (d.in / 8) + 4 * kb;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (uint32_t g = g0; g < g1; ++g) {
    uint4 xa[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      xa[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff + 256 * g + 16 * m, 0, 0));
    const uint32_t vw = __builtin_amdgcn_raw_buffer_load_b32(rv, voff + 16 * g, 0, 0);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t b = vw >> (8 * m);
      uint4 vb;
      uint32_t* e = reinterpret_cast<uint32_t*>(&vb);
#pragma unroll
      for (int k = 0; k < 4; ++k)   // elements 2k, 2k + 1: +1 (0x3F80), the bit sets the sign
        e[k] = 0x3F803F80u | ((b << (15 - 2 * k)) & 0x8000u) | ((b << (30 - 2 * k)) & 0x80000000u);
      acc = mfma(xa[m], vb, acc);
    }
  }
  // C layout: lane (t = i, kb) holds batch rows 4 kb + j of the tile
  const uint32_t tt = blockIdx.y * 16 + i;
  if (tt >= T) return;
  const float sc = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(path_plane(d.s, d, p))[q]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t nn = blockIdx.x * 16 + 4 * kb + j;
    if (nn < d.batch) zpart[((size_t)ks * d.batch + nn) * T + tt] = sc * acc[j];
  }
}
// ---------------------------------------------------------------------------
// Host side.

uint32_t class_index(const MatDev& d) {
  return d.scale_fmt * 4 + (d.k == 0 ? 0 : d.k == 2 ? 1 : d.k == 4 ? 2 : 3);
}

template <int SF, int K>
void launch_gemv_nb(uint32_t nb, dim3 grid, hipStream_t s, const MatDev& d, float* P, float* zp, uint32_t nmain,
                    uint32_t passes, uint32_t nrb) {
  if (nb == 1) hipLaunchKernelGGL((k_gemv_batch<SF, K, 1>), grid, dim3(kThreads), 0, s, d, P, zp, nmain, passes, nrb);
  else if (nb == 2)
    hipLaunchKernelGGL((k_gemv_batch<SF, K, 2>), grid, dim3(kThreads), 0, s, d, P, zp, nmain, passes, nrb);
  else hipLaunchKernelGGL((k_gemv_batch<SF, K, 4>), grid, dim3(kThreads), 0, s, d, P, zp, nmain, passes, nrb);
}

template <int SF, int K>
void launch_mfma_nt(uint32_t nt, dim3 grid, hipStream_t s, const MatDev& d, float* P, float* zp, uint32_t nz,
                    uint32_t slices) {
  const dim3 block(64 * kMfmaWaves);
  if (nt == 1) hipLaunchKernelGGL((k_mfma<SF, K, 1>), grid, block, 0, s, d, P, zp, nz, slices);
  else hipLaunchKernelGGL((k_mfma<SF, K, 2>), grid, block, 0, s, d, P, zp, nz, slices);
}

template <int SF, int K>
void launch_prefill_k(dim3 grid, hipStream_t s, const MatDev& d, const PrefillShape& S, const float* zp, float* P) {
  hipLaunchKernelGGL((k_prefill<SF, K>), grid, dim3(64 * kPrefillWaves), 0, s, d, S, zp, S.zc, P);
}

int launch_reduce(const MatDev& d, const GemmShape& S, const float* zp, const float* P, uint32_t slices,
                  hipStream_t s) {
  if (hipGetLastError() != hipSuccess) return WAL_ERR_DEVICE;
  hipLaunchKernelGGL(k_reduce, dim3((d.out + 255) / 256, d.batch), dim3(256), 0, s, d, zp, P, slices, S.zc);
  return hipGetLastError() == hipSuccess ? WAL_OK : WAL_ERR_DEVICE;
}

}  // namespace

namespace wal {

int launch_gemm_valu(const wal_info& f, const MatDev& d, uint32_t batch, void* ws, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const GemmShape S = gemm_shape(f, batch);
  uint8_t* w = static_cast<uint8_t*>(ws);
  float* zp = reinterpret_cast<float*>(w + S.off_z);
  float* P = reinterpret_cast<float*>(w + S.off_p);
  const uint32_t nb = batch >= 3 ? kGemvCols : batch;
  const uint32_t nrb = (f.d.out + kWaves * kGemvRows - 1) / (kWaves * kGemvRows);
  const uint32_t nmain = S.passes * nrb * ((batch + nb - 1) / nb);
  const dim3 grid(nmain + z_blocks(d, S));
  switch (class_index(d)) {
    case 0: launch_gemv_nb<WAL_SCALE_FP16, 0>(nb, grid, s, d, P, zp, nmain, S.passes, nrb); break;
    case 1: launch_gemv_nb<WAL_SCALE_FP16, 2>(nb, grid, s, d, P, zp, nmain, S.passes, nrb); break;
    case 2: launch_gemv_nb<WAL_SCALE_FP16, 4>(nb, grid, s, d, P, zp, nmain, S.passes, nrb); break;
    case 3: launch_gemv_nb<WAL_SCALE_FP16, 8>(nb, grid, s, d, P, zp, nmain, S.passes, nrb); break;
    case 4: launch_gemv_nb<WAL_SCALE_FP24, 0>(nb, grid, s, d, P, zp, nmain, S.passes, nrb); break;
    case 5: launch_gemv_nb<WAL_SCALE_FP24, 2>(nb, grid, s, d, P, zp, nmain, S.passes, nrb); break;
    case 6: launch_gemv_nb<WAL_SCALE_FP24, 4>(nb, grid, s, d, P, zp, nmain, S.passes, nrb); break;
    default: launch_gemv_nb<WAL_SCALE_FP24, 8>(nb, grid, s, d, P, zp, nmain, S.passes, nrb); break;
  }
  return launch_reduce(d, S, zp, P, S.passes, s);
}

int launch_gemm_mfma(const wal_info& f, const MatDev& d, uint32_t batch, void* ws, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const GemmShape S = gemm_shape(f, batch);
  uint8_t* w = static_cast<uint8_t*>(ws);
  float* zp = reinterpret_cast<float*>(w + S.off_z);
  float* P = reinterpret_cast<float*>(w + S.off_p);
  const uint32_t nt = (batch + 15) / 16;
  // one workgroup per (kMfmaTiles row tiles, kSliceCols-column slice)
  const uint32_t rblocks = (f.d.out + 16 * kMfmaTiles - 1) / (16 * kMfmaTiles), slices = S.slices;
  const uint32_t nz = z_blocks(d, S);
  const dim3 grid(nz + rblocks * slices);
  switch (class_index(d)) {
    case 0: launch_mfma_nt<WAL_SCALE_FP16, 0>(nt, grid, s, d, P, zp, nz, slices); break;
    case 1: launch_mfma_nt<WAL_SCALE_FP16, 2>(nt, grid, s, d, P, zp, nz, slices); break;
    case 2: launch_mfma_nt<WAL_SCALE_FP16, 4>(nt, grid, s, d, P, zp, nz, slices); break;
    case 3: launch_mfma_nt<WAL_SCALE_FP16, 8>(nt, grid, s, d, P, zp, nz, slices); break;
    case 4: launch_mfma_nt<WAL_SCALE_FP24, 0>(nt, grid, s, d, P, zp, nz, slices); break;
    case 5: launch_mfma_nt<WAL_SCALE_FP24, 2>(nt, grid, s, d, P, zp, nz, slices); break;
    case 6: launch_mfma_nt<WAL_SCALE_FP24, 4>(nt, grid, s, d, P, zp, nz, slices); break;
    default: launch_mfma_nt<WAL_SCALE_FP24, 8>(nt, grid, s, d, P, zp, nz, slices); break;
  }
  return launch_reduce(d, S, zp, P, slices, s);
}

int launch_gemm_prefill(const wal_info& f, const MatDev& d, uint32_t batch, void* ws, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PrefillShape S = prefill_shape(f, batch);
  uint8_t* w = static_cast<uint8_t*>(ws);
  float* zp = reinterpret_cast<float*>(w);
  float* P = S.nsplit > 1 ? reinterpret_cast<float*>(w + S.off_p) : nullptr;
  if (d.terms) {
    const dim3 zg((batch + 15) / 16, (d.terms + 15) / 16, S.zc);
    hipLaunchKernelGGL(k_zmma, zg, dim3(64), 0, s, d, zp, S.zgroups);
    if (hipGetLastError() != hipSuccess) return WAL_ERR_DEVICE;
  }
  const dim3 grid(8 * S.per_xcd);
  switch (class_index(d)) {
    case 0: launch_prefill_k<WAL_SCALE_FP16, 0>(grid, s, d, S, zp, P); break;
    case 1: launch_prefill_k<WAL_SCALE_FP16, 2>(grid, s, d, S, zp, P); break;
    case 2: launch_prefill_k<WAL_SCALE_FP16, 4>(grid, s, d, S, zp, P); break;
    case 3: launch_prefill_k<WAL_SCALE_FP16, 8>(grid, s, d, S, zp, P); break;
    case 4: launch_prefill_k<WAL_SCALE_FP24, 0>(grid, s, d, S, zp, P); break;
    case 5: launch_prefill_k<WAL_SCALE_FP24, 2>(grid, s, d, S, zp, P); break;
    case 6: launch_prefill_k<WAL_SCALE_FP24, 4>(grid, s, d, S, zp, P); break;
    default: launch_prefill_k<WAL_SCALE_FP24, 8>(grid, s, d, S, zp, P); break;
  }
  if (hipGetLastError() != hipSuccess) return WAL_ERR_DEVICE;
  if (S.nsplit == 1) return WAL_OK;
  hipLaunchKernelGGL(k_reduce, dim3((d.out + 255) / 256, batch), dim3(256), 0, s, d, zp, P, S.nsplit, S.zc);
  return hipGetLastError() == hipSuccess ? WAL_OK : WAL_ERR_DEVICE;
}

}  // namespace wal
