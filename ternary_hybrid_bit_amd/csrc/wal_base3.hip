// Base-3 stream kernels of libwal for gfx950: the packed product when T is
// stored five trits per byte (WAL2-Ternary-27B card, "Что означает битность":
// 8/5 = 1.6 bits per trit), packed continuously along each row, with fp24
// (RC1 card, "Representation": 24-bit float scales decoded to fp32) or fp16
// group scales, k sites per group and up to four binary low-rank paths.
//
// Layout of the work (bf16 activations):
//  * A pass covers 5120 trits of a row: each lane loads 16 bytes = 80 trits
//    with one buffer load, so a wavefront reads 1 KB per row, coalesced.
//  * Trits: an LDS table maps a byte to its five trits as 2-bit codes placed
//    where a mask (and a shift by 2 or 4) turns them into bf16 pairs of
//    +-2.0 / 0, the same sign-select form as the 2-bit kernels, fed to
//    v_dot2_f32_bf16 against the lane's x pairs.  Each lane reads its own
//    copy of the table (32 copies, one per LDS bank), so lookups never
//    conflict.
//  * Groups: 80 trits do not align with 128-trit groups.  Within every lane
//    a group boundary can only fall 16, 32, 48 or 64 trits in, so every lane
//    also forms the prefix sums at those four points (six extra dot
//    products, masked where a boundary cuts a byte) and keeps the one its own
//    boundary needs: the lane's part of its first group S_A, and of the next
//    group total - S_A, each scaled by its group's alpha.
//  * fp24 / fp16 scales are read through aligned dword windows and extracted
//    with v_alignbyte_b32; sites, rows, low rank and y follow the 2-bit
//    kernels (site table in LDS, transposed row butterfly, y staged in LDS).
#include <hip/hip_runtime.h>

#include "wal_device.h"
#include "wal_internal.h"

namespace {

constexpr uint32_t kGroups3 = kPassBase3 / 128;   // 40 groups per pass
constexpr uint32_t kSegRows3 = 1024;              // rows of a segment (y staged in LDS)
constexpr uint32_t kLutCopies = 32;
constexpr int kRB3 = 2;                           // rows per batch

struct Smem3 {
  float tbl[(kGroups3 + 1) * 256];     // site table [group][site byte]; slot 40 stays zero
  uint32_t lut[256 * kLutCopies];      // [byte][copy]: five trits as positioned 2-bit codes
  float z[kMaxTerms];
  float ybuf[kSegRows3 + 64];
};

// Table entry of a base-3 byte b = sum_i d_i 3^i (d = trit + 1): the 2-bit
// code of trit i (0 -> 00, +1 -> 01, -1 -> 11) at bits 14/30/12/28/10 for
// i = 0..4, so that e & 0xC000C000 holds trits (0, 1), (e << 2) & 0xC000C000
// trits (2, 3) and (e << 4) & 0xC000C000 trit 4.  Bytes above 242 map to 0.
__device__ __forceinline__ uint32_t base3_entry(uint32_t b) {
  if (b > 242) return 0;
  const uint32_t pos[5] = {14, 30, 12, 28, 10};
  uint32_t e = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t d = b % 3;
    b /= 3;
    const uint32_t code = d == 0 ? 3u : d - 1;   // t = d - 1 in two's-complement low bits
    e |= code << pos[i];
  }
  return e;
}

// The lane's 80 activation columns of a pass as bf16 pairs matching the
// operands of each byte m: P[3m] = (x[5m], x[5m+1]), P[3m+1] = (x[5m+2],
// x[5m+3]), P[3m+2] = (x[5m+4], 0); Q15 = (x[15], 0) and Q47 = (x[47], 0)
// are the parts of bytes 3 and 9 before a group boundary.
struct XLane3 {
  uint32_t P[48];
  uint32_t Q15, Q47;

  // The lane's 80 columns as loaded: bf16 pairs in column order.
  struct Raw {
    uint32_t w[40];
  };

  // Columns c0 .. c0 + 79 through a resource over x: columns past the row's
  // end (the last pass's tail) read zeros.
  static __device__ __forceinline__ void load_raw(__amdgpu_buffer_rsrc_t rx, uint32_t c0, Raw& r) {
#pragma unroll
    for (int q = 0; q < 10; ++q) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rx, 2 * c0 + 16 * q, 0, 0);
      r.w[4 * q] = v[0]; r.w[4 * q + 1] = v[1]; r.w[4 * q + 2] = v[2]; r.w[4 * q + 3] = v[3];
    }
  }

  // The same columns from activations staged in LDS (element e on).
  static __device__ __forceinline__ void load_lds(const void* xs, uint32_t e, Raw& r) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xs) + e);
#pragma unroll
    for (int q = 0; q < 10; ++q) {
      const uint4 v = src[q];
      r.w[4 * q] = v.x; r.w[4 * q + 1] = v.y; r.w[4 * q + 2] = v.z; r.w[4 * q + 3] = v.w;
    }
  }

  __device__ __forceinline__ void set(const Raw& r) {
    auto xv = [&](int j) { return (r.w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu; };
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      P[3 * m] = xv(5 * m) | (xv(5 * m + 1) << 16);
      P[3 * m + 1] = xv(5 * m + 2) | (xv(5 * m + 3) << 16);
      P[3 * m + 2] = xv(5 * m + 4);
    }
    Q15 = xv(15);
    Q47 = xv(47);
  }
};

__device__ __forceinline__ float dot2(uint32_t op, uint32_t xp, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, op), __builtin_bit_cast(bf16x2_t, xp), acc,
                                         false);
}

// Trit sums of one lane and row (2x scaled): the total over its 80 trits and
// the prefix sums up to trits 16, 32, 48 and 64.
struct Sums3 {
  float total, p16, p32, p48, p64;
};

__device__ __forceinline__ Sums3 base3_sums(const u32x4_t& c, const uint32_t* lut, const XLane3& xl) {
  constexpr uint32_t M = 0xC000C000u;
  uint32_t e[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const uint32_t b = (c[m >> 2] >> (8 * (m & 3))) & 0xFFu;
    e[m] = lut[b * kLutCopies];
  }
  float a0 = 0.f, a1 = 0.f;
  Sums3 S;
#pragma unroll
  for (int m = 0; m < 16; m += 2) {
    const uint64_t q = ((uint64_t)e[m + 1] << 32) | e[m];
    const uint64_t q2 = shl64<2>(q), q4 = shl64<4>(q);
    const uint32_t op01[2] = {e[m] & M, e[m + 1] & M};
    const uint32_t op23[2] = {(uint32_t)q2 & M, (uint32_t)(q2 >> 32) & M};
    const uint32_t op4[2] = {(uint32_t)q4 & M, (uint32_t)(q4 >> 32) & M};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = m + h;
      // prefix sums at the group boundaries a lane can hold
      if (k == 3) S.p16 = dot2(op01[h], xl.Q15, a0 + a1);
      if (k == 6) S.p32 = dot2(op01[h], xl.P[3 * k], a0 + a1);
      if (k == 9) S.p48 = dot2(op23[h], xl.Q47, dot2(op01[h], xl.P[3 * k], a0 + a1));
      if (k == 12) S.p64 = dot2(op23[h], xl.P[3 * k + 1], dot2(op01[h], xl.P[3 * k], a0 + a1));
      float& a = h ? a1 : a0;
      a = dot2(op01[h], xl.P[3 * k], a);
      a = dot2(op23[h], xl.P[3 * k + 1], a);
      a = dot2(op4[h], xl.P[3 * k + 2], a);
    }
  }
  S.total = a0 + a1;
  return S;
}

// Scale window of one row: SW dwords holding the lane's scale bytes.
template <int SF> struct Win;
template <> struct Win<WAL_SCALE_FP24> { u32x3_t w; };
template <> struct Win<WAL_SCALE_FP16> { u32x2_t w; };

template <int SF>
__device__ __forceinline__ Win<SF> load_win(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  Win<SF> W;
  if constexpr (SF == WAL_SCALE_FP24) W.w = __builtin_bit_cast(u32x3_t, __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, kStream));
  else W.w = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStream));
  return W;
}

// Scale whose first byte sits `o` bytes into the dword pair (lo, hi), as fp32.
template <int SF>
__device__ __forceinline__ float scale_at(uint32_t hi, uint32_t lo, uint32_t o) {
  const uint32_t bits = __builtin_amdgcn_alignbyte(hi, lo, o);
  if constexpr (SF == WAL_SCALE_FP24) return __uint_as_float(bits << 8);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

struct Raw3 {
  u32x4_t c;
  uint32_t sa[3];   // alpha window (fp16 uses two dwords)
  uint32_t sb[2];   // beta window (fp16 uses one dword)
  uint32_t s[2];    // site bytes of the lane's site group
};

template <int RB>
struct Batch3 {
  Raw3 r[RB];
};

// The activations of a thread's share of one pass's signed site table
// (2x scaled bf16): items e = threadIdx.x + 256 i < (kGroups3 + 1) * 16, each
// 8 columns of group e >> 4, loaded before the set-up barrier and stored
// after it.  Groups past the row's end read as zero; slot kGroups3 is zero.
struct TableX3 {
  static constexpr int kItems = ((kGroups3 + 1) * 16 + kThreads - 1) / kThreads;
  u32x4_t w[kItems];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rx, uint32_t col0) {
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const uint32_t e = threadIdx.x + kThreads * i, g = e >> 4;
      const uint32_t col = col0 + g * 128 + (e & 15) * 8;
      // the zero slot (and items past it) load from far out of range: zeros
      w[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, g < kGroups3 ? 2 * col : 0x7FFFFFF0u, 0, 0);
    }
  }

  __device__ __forceinline__ void store(float* tbl) const {
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const uint32_t e = threadIdx.x + kThreads * i;
      if (e >= (kGroups3 + 1) * 16) break;
      const uint32_t g = e >> 4, q = e & 15;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = 2.0f * __uint_as_float((j & 1) ? (w[i][j >> 1] & 0xFFFF0000u) : (w[i][j >> 1] << 16));
      float4* pos = reinterpret_cast<float4*>(tbl + g * 256 + q * 8);
      float4* neg = reinterpret_cast<float4*>(tbl + g * 256 + 128 + q * 8);
      pos[0] = make_float4(v[0], v[1], v[2], v[3]);
      pos[1] = make_float4(v[4], v[5], v[6], v[7]);
      neg[0] = make_float4(-v[0], -v[1], -v[2], -v[3]);
      neg[1] = make_float4(-v[4], -v[5], -v[6], -v[7]);
    }
  }
};

// The byte table: thread t computes byte t's entry once and writes its
// kLutCopies copies (128 contiguous bytes), starting at a thread-dependent
// 16-byte slot so that a wavefront's writes spread over the LDS banks.
__device__ __forceinline__ void build_lut(uint32_t* lut) {
  static_assert(kThreads == 256 && kLutCopies == 32, "one byte value per thread, 8 x 16 bytes of copies");
  const uint32_t e = base3_entry(threadIdx.x);
  uint4* dst = reinterpret_cast<uint4*>(lut + threadIdx.x * kLutCopies);
#pragma unroll
  for (uint32_t k = 0; k < 8; ++k) dst[(k + threadIdx.x) & 7] = make_uint4(e, e, e, e);
}

// ZP: low-rank partials prefetched per term; lut: the workgroup's first pass,
// which also fills the byte table.
template <int SF, int K, bool ROT>
__device__ __forceinline__ void stream_rows_base3(const MatDev& d, uint32_t row0, uint32_t row1, uint32_t pass,
                                                  bool first, bool lut_first, Smem3& sm) {
  constexpr int RB = kRB3;
  constexpr int LOG = ilog2(RB);
  constexpr int SH = 6 - LOG;
  constexpr int LPR = 64 >> LOG;
  constexpr uint32_t SB = SF == WAL_SCALE_FP16 ? 2 : 3;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = wave_id();
  const uint32_t nb = (row1 - row0 + RB - 1) / RB;
  const bool has_rows = wave < nb;
  uint32_t b = wave;   // the wave's batches: wave, wave + kWaves, ...

  const uint32_t pw = min(kPassBase3, d.in - pass * kPassBase3);   // trits of this pass
  const uint32_t Gp = (pw + 127) / 128, g0 = pass * kGroups3, G = d.groups;
  // first: y starts here (the low-rank term is added after the segment's
  // last pass, by store_segment)
  const uint32_t ncols = 80 * (uint32_t)lane < pw ? min(80u, pw - 80 * lane) : 0u;

  // codes
  // one resource over the blob; plane offsets go into the vector offsets
  const __amdgpu_buffer_rsrc_t rw_ = rsrc(d.codes, d.blob_bytes);
  const uint32_t vc = pass * (kPassBase3 / 5) + 16 * (ncols ? lane : 0);
  // groups of the lane's trits: A, and A + 1 when a boundary falls inside
  const uint32_t cls = lane & 7;
  const uint32_t gA = g0 + ((5 * (uint32_t)lane) >> 3);
  const bool split = (cls == 1 || cls == 3 || cls == 4 || cls == 6) && ncols;
  const uint32_t gAc = gA < G ? gA : G - 1;
  const uint32_t gB = split && gA + 1 < G ? gA + 1 : gAc;
  // alpha window: SB-byte scales of gA and gB
  const uint32_t aoff = gAc * SB, abase = aoff & ~3u, oA = aoff - abase;
  const uint32_t aplane = (uint32_t)(d.alpha - d.codes);
  const uint32_t boff = gB * SB - abase;   // byte of gB's scale within the window (0..7)
  // beta / sites: lane l < 40 owns group g0 + l of the pass
  const bool site_lane = K > 0 && (uint32_t)lane < Gp;
  const uint32_t gs = site_lane ? g0 + lane : g0;
  uint32_t vs = 0, bbase = 0, oB = 0;
  if constexpr (K > 0) {
    vs = (uint32_t)(d.sites - d.codes) + gs * K;
    bbase = (gs * SB) & ~3u;
    oB = gs * SB - bbase;
    bbase += (uint32_t)(d.beta - d.codes);
  }
  const uint32_t tslot = site_lane ? (uint32_t)lane : kGroups3;   // zero slot for other lanes
  // prefix-sum weights: which of total / p16 / p32 / p48 / p64 is S_A
  const float w16 = split && cls == 3 ? 1.f : 0.f, w32 = split && cls == 6 ? 1.f : 0.f;
  const float w48 = split && cls == 1 ? 1.f : 0.f, w64 = split && cls == 4 ? 1.f : 0.f;
  const float wT = split ? 0.f : 1.f;
  const uint32_t* lut = sm.lut + (lane & (kLutCopies - 1));

  XLane3 xl;

  // Batches past the wave's last one read through empty resources (zeros,
  // no memory access), keeping every load unconditional.
  const __amdgpu_buffer_rsrc_t r_none = rsrc(d.codes, 0u);
  auto load_batch = [&](uint32_t bb) {
    Batch3<RB> B;
    const bool live = bb < nb;
    const __amdgpu_buffer_rsrc_t rw = live ? rw_ : r_none;
    const uint32_t base = row0 + (live ? bb : nb - 1) * RB;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const uint32_t row = min(base + i, row1 - 1);
      Raw3& r = B.r[i];
      r.c = __builtin_amdgcn_raw_buffer_load_b128(rw, vc, row * d.row_stride, kStream);
      // The scale windows may reach a few bytes past the row's scales: their
      // row offset goes in the range-checked vector offset, so bytes past
      // the blob read as zero instead of touching memory.
      const Win<SF> wa = load_win<SF>(rw, aplane + abase + row * G * SB, 0);
      r.sa[0] = wa.w[0]; r.sa[1] = wa.w[1];
      if constexpr (SF == WAL_SCALE_FP24) r.sa[2] = wa.w[2]; else r.sa[2] = 0;
      if constexpr (K > 0) {
        if constexpr (SF == WAL_SCALE_FP24) {
          const u32x2_t wb = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rw, bbase + row * G * SB, 0, kStream));
          r.sb[0] = wb[0]; r.sb[1] = wb[1];
        } else {
          r.sb[0] = __builtin_amdgcn_raw_buffer_load_b32(rw, bbase + row * G * SB, 0, kStream);
          r.sb[1] = 0;
        }
        if constexpr (K == 8) {
          const u32x2_t sv = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rw, vs, row * G * K, kStream));
          r.s[0] = sv[0]; r.s[1] = sv[1];
        }
        if constexpr (K == 4) { r.s[0] = __builtin_amdgcn_raw_buffer_load_b32(rw, vs, row * G * K, kStream); r.s[1] = 0; }
        if constexpr (K == 2) { r.s[0] = __builtin_amdgcn_raw_buffer_load_b16(rw, vs, row * G * K, kStream); r.s[1] = 0; }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    return B;
  };

  auto finish_batch = [&](const Batch3<RB>& B, uint32_t bb) {
    float acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const Raw3& r = B.r[i];
      const Sums3 S = base3_sums(r.c, lut, xl);
      const float sA = wT * S.total + w16 * S.p16 + w32 * S.p32 + w48 * S.p48 + w64 * S.p64;
      // the lane's two group scales out of the window
      const float aA = scale_at<SF>(r.sa[1], r.sa[0], oA);
      const float aB = boff < 4 ? scale_at<SF>(r.sa[1], r.sa[0], boff)
                                : scale_at<SF>(r.sa[2], r.sa[1], boff - 4);
      float v = aA * sA;
      v = __builtin_fmaf(aB, S.total - sA, v);
      if constexpr (K > 0) {
        const float* tb = sm.tbl + tslot * 256;
        float sr = 0.f;
#pragma unroll
        for (int j = 0; j < K; ++j) sr += tb[(r.s[j >> 2] >> (8 * (j & 3))) & 0xFFu];
        const float bt = scale_at<SF>(r.sb[1], r.sb[0], oB);
        v = __builtin_fmaf(bt, sr, v);
      }
      acc[i] = v;
    }
    float v = treduce<RB>(acc, lane) * 0.5f;
    const uint32_t yi = bb * RB + ((uint32_t)lane >> SH);
    if (!first) v = sm.ybuf[yi] + v;
    const uint32_t row = row0 + yi;
    if ((lane & (LPR - 1)) == 0 && row < row1) sm.ybuf[yi] = v;
  };

  // Set-up loads first (L2 hits: x, the table's x), then the first two
  // batches (HBM): loads complete in order, so waiting for the set-up data
  // does not wait for the batches.
  // A rotated product (ROT) instead has the workgroup rotate the pass's 40
  // groups (RotPass: three 16-group tiles, the groups past the pass load
  // zeros, so the table's zero slot receives zeros); the pass then goes
  // through LDS twice, as compact activations that each lane reads its
  // columns from, and as the table.
  const __amdgpu_buffer_rsrc_t rx = x_rsrc<WAL_X_BF16>(d.x, d.in);
  RotPass<WAL_X_BF16, kGroups3> rp;
  XLane3::Raw xr;
  TableX3 tx;
  if constexpr (ROT) {
    rp.load(rx, pass * kPassBase3);
  } else {
    XLane3::load_raw(rx, pass * kPassBase3 + 80 * lane, xr);
    if constexpr (K > 0) tx.load(rx, pass * kPassBase3);
  }
  Batch3<RB> B0 = load_batch(b);
  Batch3<RB> B1 = load_batch(b + kWaves);
  if constexpr (ROT) rp.compute();

  __syncthreads();   // readers of the previous table are done
  if (lut_first) build_lut(sm.lut);
  if constexpr (ROT) {
    rp.store_x(sm.tbl);
    __syncthreads();
    XLane3::load_lds(sm.tbl, 80 * lane, xr);
    if constexpr (K > 0) {
      __syncthreads();   // every lane has its columns
      rp.store_tbl(sm.tbl, kGroups3 + 1);
    }
  } else if constexpr (K > 0) {
    tx.store(sm.tbl);
  }
  __syncthreads();
  if (!has_rows) return;
  xl.set(xr);

  for (;;) {
    const Batch3<RB> B2 = load_batch(b + 2 * kWaves);
    finish_batch(B0, b);
    if (b + kWaves >= nb) break;
    b += kWaves;
    B0 = load_batch(b + 2 * kWaves);
    finish_batch(B1, b);
    if (b + kWaves >= nb) break;
    b += kWaves;
    B1 = load_batch(b + 2 * kWaves);
    finish_batch(B2, b);
    if (b + kWaves >= nb) break;
    b += kWaves;
  }
}

// One segment, pass by pass, then its store (store_segment: the low-rank
// term, or with P one pass's partial sums and the reduce of a completed row
// block).  With count (the workgroup's last segment) the store may count
// the workgroup finished; returns whether it did.
template <int SF, int K, class ZJ, bool ROT>
__device__ __forceinline__ bool run_segment_base3(const MatDev& d, uint32_t row0, uint32_t row1, bool lut_first,
                                                  Smem3& sm, const Fuse& f, float* P = nullptr,
                                                  uint32_t split_pass = 0, uint32_t* cnt = nullptr,
                                                  bool count = false) {
  const uint32_t npass = (d.in + kPassBase3 - 1) / kPassBase3;
  const bool split = P != nullptr;
  const uint32_t p0 = split ? split_pass : 0, p1 = split ? split_pass + 1 : npass;
  for (uint32_t pass = p0; pass < p1; ++pass)
    stream_rows_base3<SF, K, ROT>(d, row0, row1, pass, pass == p0, lut_first && pass == p0, sm);
  return store_segment<WAL_X_BF16, ZJ, ROT>(d, row0, row1, SegEnd{sm.tbl, sm.z, sm.ybuf}, f, P, split_pass, npass,
                                            cnt, count);
}

// Low-rank jobs of grouped plans and single products, as in the 2-bit
// kernels (bf16 activations).
template <bool ROT>
__device__ __forceinline__ void z_job_grouped3(const MatDev* __restrict__ descs, const uint32_t* __restrict__ jobs,
                                               uint32_t j, uint32_t terms, const uint32_t* epoch, void* xs) {
  const uint32_t m = jobs[2 * j], tc = jobs[2 * j + 1];
  const MatDev& d = descs[m];
  const uint32_t t0 = tc >> 16, cc = tc & 0xFFFFu;
  const uint32_t c0 = cc * kZChunkCols, c1 = min(d.in, c0 + kZChunkCols);
  z_job<WAL_X_BF16, ZJobsGrouped, kZOutTagged, ROT>(d, terms, t0, reinterpret_cast<uint64_t*>(d.z) + (size_t)cc * d.terms,
                                              c0, c1, epoch, xs);
}

// Two workgroups per CU (the LDS allows no more); kernels that rotate x are
// held to the registers of two wavefronts per SIMD.
constexpr int stream3_waves_per_simd(bool ROT) { return ROT ? 2 : 1; }

template <int SF, int K, bool ROT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(stream3_waves_per_simd(ROT))))
void k_stream3_grouped(const MatDev* __restrict__ descs,
                                                              const uint32_t* __restrict__ blockseg,
                                                              const Seg* __restrict__ segs,
                                                              const uint32_t* __restrict__ jobs, Fuse f) {
  __shared__ Smem3 sm;
  const uint32_t t = blockIdx.x;
  bool counted = false;
  if (t < f.nz) {
    z_job_grouped3<ROT>(descs, jobs, t, zjob_terms<ZJobsGrouped>(f), epoch_of(f), sm.tbl);
  } else {
    const uint32_t b = t - f.nz;
    const uint32_t s0 = blockseg[b], s1 = blockseg[b + 1];
    for (uint32_t s = s0; s < s1; ++s) {
      const Seg sg = segs[s];
      const MatDev& d = descs[sg.mat];
      if (sg.pass1)
        counted = run_segment_base3<SF, K, ZJobsGrouped, ROT>(d, sg.row0, sg.row1, s == s0, sm, f, d.P,
                                                              sg.pass1 - 1, f.sync + d.cnt_off, s + 1 == s1);
      else
        counted = run_segment_base3<SF, K, ZJobsGrouped, ROT>(d, sg.row0, sg.row1, s == s0, sm, f, nullptr, 0,
                                                              nullptr, s + 1 == s1);
    }
  }
  if (!counted) finish_launch(f);
}

template <int SF, int K, bool ROT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(stream3_waves_per_simd(ROT))))
void k_stream3_single(MatDev d, uint32_t rows_per_block, uint32_t nrb,
                                                             float* P, uint32_t* cnt, Fuse f) {
  // block t < f.nz: low-rank job t; else without P block b takes rows
  // [b rpb, b rpb + rpb) over every pass, with P pass b / nrb of row block
  // b % nrb
  __shared__ Smem3 sm;
  const uint32_t t = blockIdx.x;
  bool counted = false;
  if (t < f.nz) {
    const uint32_t tcs = (d.terms + kZTerms - 1) / kZTerms, tc = t % tcs, cc = t / tcs;
    const uint32_t c0 = cc * kZSingleCols, c1 = min(d.in, c0 + kZSingleCols);
    z_chunk_rot<WAL_X_BF16, (int)kZTerms, kZOutTagged, ROT>(d, tc * kZTerms,
                                                       reinterpret_cast<uint64_t*>(d.z) + (size_t)cc * d.terms, c0,
                                                       c1, epoch_of(f), sm.tbl);
  } else {
    const uint32_t b = t - f.nz;
    const uint32_t rb = P ? b % nrb : b;
    const uint32_t r0 = rb * rows_per_block;
    const uint32_t r1 = min(d.out, r0 + rows_per_block);
    if (r0 < r1)
      counted = run_segment_base3<SF, K, ZJobsSingle, ROT>(d, r0, r1, true, sm, f, P, P ? b / nrb : 0u, cnt, true);
  }
  if (!counted) finish_launch(f);
}

}  // namespace

namespace wal {

template <bool ROT>
GroupedFn base3_grouped(uint32_t cls) {
  switch (cls & 7) {
    case 0: return k_stream3_grouped<WAL_SCALE_FP16, 0, ROT>;
    case 1: return k_stream3_grouped<WAL_SCALE_FP16, 2, ROT>;
    case 2: return k_stream3_grouped<WAL_SCALE_FP16, 4, ROT>;
    case 3: return k_stream3_grouped<WAL_SCALE_FP16, 8, ROT>;
    case 4: return k_stream3_grouped<WAL_SCALE_FP24, 0, ROT>;
    case 5: return k_stream3_grouped<WAL_SCALE_FP24, 2, ROT>;
    case 6: return k_stream3_grouped<WAL_SCALE_FP24, 4, ROT>;
    default: return k_stream3_grouped<WAL_SCALE_FP24, 8, ROT>;
  }
}

template <bool ROT>
SingleFn base3_single(uint32_t cls) {
  switch (cls & 7) {
    case 0: return k_stream3_single<WAL_SCALE_FP16, 0, ROT>;
    case 1: return k_stream3_single<WAL_SCALE_FP16, 2, ROT>;
    case 2: return k_stream3_single<WAL_SCALE_FP16, 4, ROT>;
    case 3: return k_stream3_single<WAL_SCALE_FP16, 8, ROT>;
    case 4: return k_stream3_single<WAL_SCALE_FP24, 0, ROT>;
    case 5: return k_stream3_single<WAL_SCALE_FP24, 2, ROT>;
    case 6: return k_stream3_single<WAL_SCALE_FP24, 4, ROT>;
    default: return k_stream3_single<WAL_SCALE_FP24, 8, ROT>;
  }
}

GroupedFn base3_grouped_kernel(uint32_t cls, bool rot) { return rot ? base3_grouped<true>(cls) : base3_grouped<false>(cls); }
SingleFn base3_single_kernel(uint32_t cls, bool rot) { return rot ? base3_single<true>(cls) : base3_single<false>(cls); }

uint32_t base3_seg_rows() { return kSegRows3; }

}  // namespace wal
