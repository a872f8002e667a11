// gfx950 (CDNA4) kernels and the product entry points of libwal.
//
// Operator (WAL-Ternary-8B cards, "Модель пішімі" / "Representation"):
//     y = (alpha * T + beta * R) x + sum_p U_p diag(s_p) V_p^T x
// computed straight from the packed planes described in include/wal.h.
//
// Kernels:
//  * the binary low-rank reductions z_p[r] = s_p[r] * sum_j (-1)^{V bit} x_j,
//    a pre-pass into the caller's workspace: kZTerms terms per workgroup for
//    grouped products (k_z_grouped), kZTerms terms x 4096 columns per
//    workgroup for a single product (k_z_chunks, partial sums that the
//    streaming kernel adds), so that wide matrices get enough workgroups.
//  * k_stream_*: one streaming pass over the packed planes.  Every workgroup
//    owns a contiguous range of rows of one or more matrices (for grouped
//    products the host splits the total packed bytes evenly over a grid that
//    fits the GPU at once, so no workgroup waits for another).  Inside a
//    range, the 4 wavefronts take batches of RB rows in turn:
//      - codes: each lane owns 64 consecutive columns of a 4096-column pass
//        and reads its 16 bytes of 2-bit codes per row with one buffer load,
//        so a wavefront reads a 1 KB row segment fully coalesced.  Row
//        offsets live in scalar registers (buffer soffset), so stepping rows
//        costs no vector instructions.  The loads of the next batch are in
//        flight while the current batch is computed.
//      - trits: a code keeps its magnitude bit below its sign bit, so shifting
//        a dword to put a code pair at bits 14-15 and 30-31 and masking with
//        0xC000C000 gives a bf16 pair whose halves are +-2.0 or 0: the trits
//        become sign-selected copies of x with no multiply and no table, and
//        v_dot2_f32_bf16 adds both into fp32 (products by +-2 and 0 are
//        exact).  The lane's x stays in registers for the whole pass.
//      - sites: an LDS table per workgroup holds +2x and -2x for every
//        position of every group of the pass ([group][256] floats), so a site
//        byte (7-bit position, sign in bit 7) indexes its signed value.
//      - scales: alpha multiplies the lane's ternary partial and beta its site
//        partial once per row in fp32 (fp16 scales feed v_fma_mix directly).
//      - rows: the RB row partials of a lane are reduced across the
//        wavefront with one transposed butterfly (permlane swaps and DPP), so
//        each row's total lands in 64/RB lanes; those lanes add the low-rank
//        term sum_t (-1)^{U bit} z_t (one term per lane) and one of them
//        stores y.  Matrices wider than one pass accumulate y pass by pass.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <atomic>
#include <cstring>
#include <new>

#include "wal_device.h"
#include "wal_internal.h"

using namespace wal;

namespace {

// ---------------------------------------------------------------------------
// A lane's 64 activation columns of one pass, held in registers.
template <int XT> struct XLane;

template <> struct XLane<WAL_X_BF16> {
  // p[8d + i] = bf16 pair (x[c + 16d + i], x[c + 16d + 8 + i]): the pair of
  // columns whose codes sit at bits 2i and 2i + 16 of the lane's dword d.
  uint32_t p[32];
  static constexpr float kHalf = 0.5f;   // decoded trits and table entries are 2x

  // The lane's 64 columns as loaded: bf16 pairs in column order.
  struct Raw {
    uint32_t w[32];
  };

  // Columns c .. c + 63 through a resource over x (lanes past the pass width
  // read zeros).
  static __device__ __forceinline__ void load_raw(__amdgpu_buffer_rsrc_t rx, uint32_t c, Raw& r) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rx, 2 * c + 16 * q, 0, 0);
      r.w[4 * q] = v[0]; r.w[4 * q + 1] = v[1]; r.w[4 * q + 2] = v[2]; r.w[4 * q + 3] = v[3];
    }
  }

  __device__ __forceinline__ void set(const Raw& r) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int lo = 16 * d + i, hi = 16 * d + 8 + i;
        const uint32_t xl = (r.w[lo >> 1] >> (16 * (lo & 1))) & 0xFFFFu;
        const uint32_t xh = (r.w[hi >> 1] >> (16 * (hi & 1))) & 0xFFFFu;
        p[8 * d + i] = xl | (xh << 16);
      }
  }

  // 2 * sum_j T_j x_j over the lane's 64 columns of one row.  One 64-bit
  // shift positions the code pairs of two dwords at once (a full-rate
  // instruction on gfx950, as is a 32-bit shift); the mask and the dot
  // product then work on each half.
  template <int I>
  __device__ __forceinline__ void dot_pairs(uint64_t q, int h, float& a0, float& a1) const {
    const uint64_t t = shl64<14 - 2 * I>(q);
    const uint32_t lo = (uint32_t)t & 0xC000C000u, hi = (uint32_t)(t >> 32) & 0xC000C000u;
    a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lo),
                                         __builtin_bit_cast(bf16x2_t, p[16 * h + I]), a0, false);
    a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, hi),
                                         __builtin_bit_cast(bf16x2_t, p[16 * h + 8 + I]), a1, false);
    if constexpr (I < 7) dot_pairs<I + 1>(q, h, a0, a1);
  }

  __device__ __forceinline__ float dot(const u32x4_t& c) const {
    float a0 = 0.f, a1 = 0.f;
    dot_pairs<0>(((uint64_t)c[1] << 32) | c[0], 0, a0, a1);
    dot_pairs<0>(((uint64_t)c[3] << 32) | c[2], 1, a0, a1);
    return a0 + a1;
  }
};

template <> struct XLane<WAL_X_F32> {
  float f[64];
  static constexpr float kHalf = 1.0f;

  struct Raw {
    float f[64];
  };

  static __device__ __forceinline__ void load_raw(__amdgpu_buffer_rsrc_t rx, uint32_t c, Raw& r) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rx, 4 * c + 16 * q, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) r.f[4 * q + j] = __uint_as_float(v[j]);
    }
  }

  __device__ __forceinline__ void set(const Raw& r) {
#pragma unroll
    for (int q = 0; q < 64; ++q) f[q] = r.f[q];
  }

  // sum_j T_j x_j: sign-extend each 2-bit code to {-1, 0, +1} and accumulate.
  __device__ __forceinline__ float dot(const u32x4_t& c) const {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = (int)(c[d] << (30 - 2 * i)) >> 30;
        acc[d] = __builtin_fmaf((float)t, f[16 * d + i], acc[d]);
      }
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
};

// ---------------------------------------------------------------------------
// Shared memory of the streaming kernels.
struct StreamSmem {
  float tbl[32 * 256];      // [group of the pass][site byte] -> +-2x (bf16) or +-x (fp32)
  float z[kMaxTerms];       // low-rank reductions of the current matrix
  float ybuf[kSegRows + 64];   // y of the segment's rows, accumulated over passes
                               // (padded: lanes of a last, partial batch index past it)
};

// The activations of a thread's share of one 4096-column pass's signed table:
// items e = threadIdx.x and threadIdx.x + 256, each 8 columns of group e >> 4.
// They are loaded before the set-up barrier and stored after it; columns past
// the row's end (groups past the pass width) read as zero.
template <int XT>
struct TableX {
  static constexpr int kW = XT == WAL_X_BF16 ? 4 : 8;   // dwords per item
  uint32_t w[2][kW];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rx, uint32_t col0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t e = threadIdx.x + kThreads * i;
      const uint32_t col = col0 + (e >> 4) * 128 + (e & 15) * 8;
#pragma unroll
      for (int h = 0; h < kW / 4; ++h) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rx, col * (XT == WAL_X_BF16 ? 2 : 4) + 16 * h, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) w[i][4 * h + j] = v[j];
      }
    }
  }

  // +-2x (bf16 x) or +-x (fp32 x) for every position of every group:
  // tbl[group][site byte].
  __device__ __forceinline__ void store(float* tbl) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t e = threadIdx.x + kThreads * i;
      const uint32_t g = e >> 4, q = e & 15;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (XT == WAL_X_BF16)
          v[j] = 2.0f * __uint_as_float((j & 1) ? (w[i][j >> 1] & 0xFFFF0000u) : (w[i][j >> 1] << 16));
        else
          v[j] = __uint_as_float(w[i][j]);
      }
      float4* pos = reinterpret_cast<float4*>(tbl + g * 256 + q * 8);
      float4* neg = reinterpret_cast<float4*>(tbl + g * 256 + 128 + q * 8);
      pos[0] = make_float4(v[0], v[1], v[2], v[3]);
      pos[1] = make_float4(v[4], v[5], v[6], v[7]);
      neg[0] = make_float4(-v[0], -v[1], -v[2], -v[3]);
      neg[1] = make_float4(-v[4], -v[5], -v[6], -v[7]);
    }
  }
};

// Packed data of one row for one lane.
struct RowRaw {
  u32x4_t c;        // 16 bytes of 2-bit codes (64 trits)
  uint32_t s;       // site bytes (k / 2 of them)
  uint32_t a, b;    // raw alpha, beta of the lane's group
};

template <int RB>
struct Batch {
  RowRaw r[RB];
  uint32_t u;       // U byte holding this lane's low-rank sign bit
};

// Per-pass lane constants of the 2-bit stream.
struct Lane2 {
  __amdgpu_buffer_rsrc_t rw;  // the blob from the codes plane on
  uint32_t vc, vs, va, vb;    // lane offsets (from the codes plane) in row 0 of each plane
  uint32_t sc, ss, sa;        // row strides (bytes) of each plane
  const float* tb;            // the lane's group in the site table
  const uint8_t* up;          // U byte of the lane's first low-rank term (row 0)
  uint32_t ub, ubit;          // bytes per U row, bit of the term in its byte
  bool uon;                   // the lane owns a low-rank term
};

// One pass of one segment.  The workgroup-wide set-up of the pass (site table,
// low-rank terms, behind barriers) runs after each wave has issued the loads
// of its first batch and of its x columns, so the set-up overlaps the
// memory latency instead of adding to it.  Every wave reaches both barriers.
// ZP: low-rank partials (column chunks) prefetched per term.
template <int XT, int SF, int K, int RB, int ZP>
__device__ __forceinline__ void stream_rows_2bit(const MatDev& d, uint32_t row0, uint32_t row1, uint32_t pass,
                                                 uint32_t npass, bool split, StreamSmem& sm) {
  constexpr int LOG = ilog2(RB);
  constexpr int SH = 6 - LOG;        // lane >> SH = row of the batch after the reduction
  constexpr int LPR = 64 >> LOG;     // lanes per row after the reduction
  constexpr uint32_t SB = SF == WAL_SCALE_FP16 ? 2 : 3;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = wave_id();
  const uint32_t nb = (row1 - row0 + RB - 1) / RB;
  const bool has_rows = wave < nb;
  uint32_t b = wave;   // the wave's batches: wave, wave + kWaves, ...

  const uint32_t pw = min(kPass2bit, d.in - pass * kPass2bit);
  const uint32_t Gp = pw / 128, g0 = pass * (kPass2bit / 128), G = d.groups;
  const bool on = (uint32_t)lane < 2 * Gp;
  const uint32_t gl = on ? (uint32_t)lane >> 1 : 0;
  // first: y starts here (no earlier pass in LDS); last: the low-rank term is
  // added here.  A split pass (one pass of a row range, written as a partial
  // sum) is both first and without the low-rank term.
  const bool first = split || pass == 0, last = !split && pass + 1 == npass;

  // One resource over the blob; the plane offsets go into the per-lane
  // offsets (the planes are 256-byte aligned, so alignments carry over).
  Lane2 L;
  L.rw = rsrc(d.codes, d.blob_bytes);
  L.vc = pass * (kPass2bit / 4) + 16 * (on ? lane : 0);
  L.sc = d.row_stride;
  L.va = (uint32_t)(d.alpha - d.codes) + (g0 + gl) * SB;
  L.sa = G * SB;
  if constexpr (K > 0) {
    L.vb = (uint32_t)(d.beta - d.codes) + (g0 + gl) * SB;
    L.vs = (uint32_t)(d.sites - d.codes) + (g0 + gl) * K + (lane & 1) * (K / 2);
    L.ss = G * K;
  }
  L.tb = sm.tbl + ((uint32_t)lane >> 1) * 256;
  const uint32_t ti = lane & (LPR - 1);
  L.uon = last && ti < d.terms;
  L.ub = (d.rank + 7) / 8;
  L.up = d.codes;    // any readable byte for lanes without a low-rank term
  L.ubit = 0;
  if (L.uon) {
    const uint32_t p = ti / d.rank, r = ti % d.rank;
    L.up = path_plane(d.U, d, p) + r / 8;
    L.ubit = r & 7;
  }
  // The U bytes go through buffer instructions too (a generic pointer would
  // need flat instructions, whose completion the compiler tracks more
  // conservatively).  Passes that need no U bits (all but the last) read
  // them through an empty resource.
  const uint32_t uoff = (uint32_t)(L.up - d.codes);
  const uint32_t ustride = L.uon ? L.ub : 0;
  const bool ulive = last && d.terms;

  XLane<XT> xl;

  // Every load is unconditional (rows past the range repeat the last row of
  // the range), so the compiler never has to merge loaded and unloaded
  // values, which would make it wait for every load in flight.  Batches past
  // the wave's last one (the prefetch at the end of the loop) read through
  // empty resources: out-of-range buffer loads return 0 without a memory
  // access, and the instruction stream stays the same.
  // (Out-of-range buffer loads return 0 without a memory access.)
  const __amdgpu_buffer_rsrc_t r_none = rsrc(d.codes, 0u);
  auto load_batch = [&](uint32_t bb) {
    Batch<RB> B;
    const bool live = bb < nb;
    const __amdgpu_buffer_rsrc_t rw = live ? L.rw : r_none;
    const __amdgpu_buffer_rsrc_t ru = live && ulive ? L.rw : r_none;
    const uint32_t base = row0 + (live ? bb : nb - 1) * RB;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const uint32_t row = min(base + i, row1 - 1);
      RowRaw& r = B.r[i];
      r.c = __builtin_amdgcn_raw_buffer_load_b128(rw, L.vc, row * L.sc, kStream);
      r.a = load_scale<SF>(rw, L.va, row * L.sa);
      if constexpr (K == 8) r.s = __builtin_amdgcn_raw_buffer_load_b32(rw, L.vs, row * L.ss, kStream);
      if constexpr (K == 4) r.s = __builtin_amdgcn_raw_buffer_load_b16(rw, L.vs, row * L.ss, kStream);
      if constexpr (K == 2) r.s = __builtin_amdgcn_raw_buffer_load_b8(rw, L.vs, row * L.ss, kStream);
      if constexpr (K > 0) r.b = load_scale<SF>(rw, L.vb, row * L.sa);
    }
    const uint32_t ry = min(base + ((uint32_t)lane >> SH), row1 - 1);
    B.u = __builtin_amdgcn_raw_buffer_load_b8(ru, uoff + ry * ustride, 0, kStream);
    // keep the scheduler from sinking these loads into the next computation
    __builtin_amdgcn_sched_barrier(0);
    return B;
  };

  auto finish_batch = [&](const Batch<RB>& B, uint32_t bb) {
    float acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const RowRaw& r = B.r[i];
      float v = scale_fma<SF>(r.a, xl.dot(r.c), 0.f);
      if constexpr (K > 0) {
        float sr = L.tb[r.s & 0xFFu];
#pragma unroll
        for (int j = 1; j < K / 2; ++j) sr += L.tb[(r.s >> (8 * j)) & 0xFFu];
        v = scale_fma<SF>(r.b, sr, v);
      }
      acc[i] = v;
    }
    float v = treduce<RB>(acc, lane) * XLane<XT>::kHalf;
    const uint32_t yi = bb * RB + ((uint32_t)lane >> SH);   // row within the segment
    if (!first) v = sm.ybuf[yi] + v;   // written by this lane in the previous pass
    const uint32_t base = row0 + bb * RB;
    const uint32_t row = base + ((uint32_t)lane >> SH);
    if (last && d.terms) {
      float c = 0.f;
      if (L.uon) {
        const float zt = sm.z[ti];
        c = ((B.u >> L.ubit) & 1u) ? -zt : zt;
      }
      // terms beyond one per lane (more than 64 / RB of them)
      const uint32_t ry = min(row, row1 - 1);
      for (uint32_t t = ti + LPR; t < d.terms; t += LPR) {
        const uint32_t p = t / d.rank, r = t % d.rank;
        const uint32_t byte = path_plane(d.U, d, p)[(size_t)ry * L.ub + r / 8];
        const float zt = sm.z[t];
        c += ((byte >> (r & 7)) & 1u) ? -zt : zt;
      }
      v += group_sum<LPR>(c);
    }
    if ((lane & (LPR - 1)) == 0 && row < row1)
      sm.ybuf[yi] = v;
  };

  // Set-up loads first: the lane's x, the x of its share of the site table
  // and the low-rank partials (L2 hits).  Vector memory loads complete in
  // order, so waiting for these after the first batch's loads (HBM) are
  // issued does not wait for the batch.
  const __amdgpu_buffer_rsrc_t rx = x_rsrc<XT>(d.x, d.in);
  typename XLane<XT>::Raw xr;
  XLane<XT>::load_raw(rx, pass * kPass2bit + 64 * lane, xr);
  TableX<XT> tx;
  if constexpr (K > 0) tx.load(rx, pass * kPass2bit);
  const bool zpass = !split && pass == 0 && d.terms;
  ZPart<ZP> zp;
  if (zpass) z_prefetch<ZP>(d, threadIdx.x, zp);

  // Two batches in registers: while one is reduced, the next is in flight
  // (three resident workgroups per CU keep three wavefronts per SIMD, six
  // batches, in flight).
  Batch<RB> B0 = load_batch(b);

  __syncthreads();   // readers of the previous table and z are done
  if (zpass && threadIdx.x < d.terms) sm.z[threadIdx.x] = z_total<ZP>(d, threadIdx.x, zp);
  if constexpr (K > 0) tx.store(sm.tbl);
  __syncthreads();
  if (!has_rows) return;
  xl.set(xr);

  for (;;) {
    const Batch<RB> B1 = load_batch(b + kWaves);
    finish_batch(B0, b);
    if (b + kWaves >= nb) break;
    b += kWaves;
    B0 = load_batch(b + kWaves);
    finish_batch(B1, b);
    if (b + kWaves >= nb) break;
    b += kWaves;
  }
}

// One segment (rows row0..row1-1 of one matrix) of a workgroup, pass by pass.
// SF and K are the matrix's scale format and sites per group: every
// (scale format, k) class has kernels of its own, so the registers of the
// hot fp16 / k = 8 loop are not set by the heavier fp24 loads.
// With P, only pass `split_pass`, written to P[split_pass][row] without the
// low-rank term (a reduce adds the passes and that term).
template <int XT, int SF, int K, int RB, int ZP>
__device__ __forceinline__ void run_segment_2bit(const MatDev& d, uint32_t row0, uint32_t row1, StreamSmem& sm,
                                                 float* P = nullptr, uint32_t split_pass = 0) {
  const uint32_t npass = (d.in + kPass2bit - 1) / kPass2bit;
  const bool split = P != nullptr;
  const uint32_t p0 = split ? split_pass : 0, p1 = split ? split_pass + 1 : npass;
  for (uint32_t pass = p0; pass < p1; ++pass)
    stream_rows_2bit<XT, SF, K, RB, ZP>(d, row0, row1, pass, npass, split, sm);
  // y leaves through LDS: one coalesced write of the segment's rows instead
  // of a few scattered bytes per batch of rows.
  __syncthreads();
  const uint32_t nrows = row1 - row0;
  float* dst = split ? P + (size_t)split_pass * d.out : d.y;
  for (uint32_t i = threadIdx.x; i < nrows; i += kThreads) dst[row0 + i] = sm.ybuf[i];
}

// Three workgroups per CU (the LDS of a workgroup allows it) when the class's
// registers fit three wavefronts per SIMD without spilling; the fp32 and the
// fp24 / k = 8 loops need more registers and run two.
constexpr int stream_waves_per_simd(int XT, int SF, int K) {
  return XT == WAL_X_BF16 && !(SF == WAL_SCALE_FP24 && K == 8) ? 3 : 1;
}

template <int XT, int SF, int K, int RB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(stream_waves_per_simd(XT, SF, K))))
void k_stream_grouped(const MatDev* __restrict__ descs, const uint32_t* __restrict__ blockseg,
                      const Seg* __restrict__ segs) {
  __shared__ StreamSmem sm;
  const uint32_t s0 = blockseg[blockIdx.x], s1 = blockseg[blockIdx.x + 1];
  for (uint32_t s = s0; s < s1; ++s) {
    const Seg sg = segs[s];
    run_segment_2bit<XT, SF, K, RB, kZSinglePrefetch>(descs[sg.mat], sg.row0, sg.row1, sm);
  }
}

template <int XT, int SF, int K, int RB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(stream_waves_per_simd(XT, SF, K))))
void k_stream_single(MatDev d, uint32_t rows_per_block, uint32_t nrb, float* P) {
  // without P: block b takes rows [b rpb, b rpb + rpb) over every pass; with
  // P: block b takes pass b / nrb of row block b % nrb
  __shared__ StreamSmem sm;
  const uint32_t rb = P ? blockIdx.x % nrb : blockIdx.x;
  const uint32_t r0 = rb * rows_per_block;
  const uint32_t r1 = min(d.out, r0 + rows_per_block);
  if (r0 < r1) run_segment_2bit<XT, SF, K, RB, kZSinglePrefetch>(d, r0, r1, sm, P, P ? blockIdx.x / nrb : 0u);
}

// Low-rank partials of a single product: block (tc, cc) computes terms
// kZTerms tc .. kZTerms tc + kZTerms - 1 over columns [8192 cc, 8192 cc + 8192)
// into d.z[cc][t].  Few terms per block keep each thread's share short: the
// streaming kernel waits for this launch.
template <int XT>
__global__ __launch_bounds__(kThreads) void k_z_chunks(MatDev d) {
  const uint32_t tcs = (d.terms + kZTerms - 1) / kZTerms;
  const uint32_t tc = blockIdx.x % tcs, cc = blockIdx.x / tcs;
  const uint32_t c0 = cc * kZSingleCols, c1 = min(d.in, c0 + kZSingleCols);
  z_chunk<XT, (int)kZTerms>(d, d.x, tc * kZTerms, d.z + (size_t)cc * d.terms, c0, c1);
}

template <int XT>
__global__ __launch_bounds__(kThreads) void k_z_grouped(const MatDev* __restrict__ descs,
                                                        const uint32_t* __restrict__ jobs) {
  const uint32_t m = jobs[2 * blockIdx.x], tc = jobs[2 * blockIdx.x + 1];
  const MatDev& d = descs[m];
  const uint32_t t0 = tc >> 16, cc = tc & 0xFFFFu;
  const uint32_t c0 = cc * kZChunkCols, c1 = min(d.in, c0 + kZChunkCols);
  z_chunk<XT, (int)kZTerms>(d, d.x, t0, d.z + (size_t)cc * d.terms, c0, c1);
}

// ---------------------------------------------------------------------------
// Host helpers.

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t xelem(int xdt) { return xdt == WAL_X_F32 ? 4 : 2; }

uint64_t up64(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

MatDev make_dev(const wal_info* f, const void* W, const void* x, float* y, float* z, uint32_t ldx,
                uint32_t ldy, uint32_t batch) {
  MatDev m{};
  const uint8_t* base = static_cast<const uint8_t*>(W);
  m.codes = base + f->off_codes;
  m.sites = f->d.k ? base + f->off_sites : m.codes;
  m.alpha = base + f->off_alpha;
  m.beta = f->d.k ? base + f->off_beta : m.alpha;
  // check_info has verified the canonical layout: path planes at a fixed stride
  const bool paths = f->d.n_paths > 0;
  m.V = paths ? base + f->off_V[0] : m.codes;
  m.U = paths ? base + f->off_U[0] : m.codes;
  m.s = paths ? base + f->off_s[0] : m.codes;
  m.pstride = f->d.n_paths > 1 ? (uint32_t)(f->off_V[1] - f->off_V[0]) : 0;
  m.x = x; m.y = y; m.z = z;
  m.out = f->d.out; m.in = f->d.in; m.k = f->d.k; m.n_paths = f->d.n_paths;
  m.rank = f->d.rank; m.scale_fmt = f->d.scale_fmt; m.row_stride = f->row_stride;
  m.groups = f->groups; m.ldx = ldx; m.ldy = ldy; m.batch = batch;
  m.terms = f->d.n_paths * f->d.rank;
  m.blob_bytes = (uint32_t)(f->total_bytes - f->off_codes);
  m.trit_fmt = f->d.trit_fmt;
  m.zc = 1;
  return m;
}

int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? WAL_OK : WAL_ERR_DEVICE;
}

constexpr int kRB = 4;   // rows per batch of the 2-bit streaming kernels
// Batch from which WAL_GEMM_AUTO takes the MFMA kernel (measured on MI355X
// on the 4096 x 12288 shape); below it the batched GEMV, and at batch 1 the
// single-product path, which is faster still.
constexpr uint32_t kGemmCrossover = 2;
constexpr uint32_t kClasses = 16;   // kernel classes (see class_of)

// Kernel class of a matrix: 8 * trit_fmt + 4 * scale_fmt + index of k in {0, 2, 4, 8}.
uint32_t class_of(const wal_desc& d) {
  return d.trit_fmt * 8 + d.scale_fmt * 4 + (d.k == 0 ? 0 : d.k == 2 ? 1 : d.k == 4 ? 2 : 3);
}

// Longest row range one workgroup of a class takes (its y is staged in LDS).
uint32_t seg_rows(uint32_t cls) { return cls >= 8 ? base3_seg_rows() : kSegRows; }

template <int XT>
GroupedFn grouped_kernel(uint32_t cls) {
  switch (cls) {
    case 0: return k_stream_grouped<XT, WAL_SCALE_FP16, 0, kRB>;
    case 1: return k_stream_grouped<XT, WAL_SCALE_FP16, 2, kRB>;
    case 2: return k_stream_grouped<XT, WAL_SCALE_FP16, 4, kRB>;
    case 3: return k_stream_grouped<XT, WAL_SCALE_FP16, 8, kRB>;
    case 4: return k_stream_grouped<XT, WAL_SCALE_FP24, 0, kRB>;
    case 5: return k_stream_grouped<XT, WAL_SCALE_FP24, 2, kRB>;
    case 6: return k_stream_grouped<XT, WAL_SCALE_FP24, 4, kRB>;
    default: return k_stream_grouped<XT, WAL_SCALE_FP24, 8, kRB>;
  }
}
template <int XT>
SingleFn single_kernel(uint32_t cls) {
  switch (cls) {
    case 0: return k_stream_single<XT, WAL_SCALE_FP16, 0, kRB>;
    case 1: return k_stream_single<XT, WAL_SCALE_FP16, 2, kRB>;
    case 2: return k_stream_single<XT, WAL_SCALE_FP16, 4, kRB>;
    case 3: return k_stream_single<XT, WAL_SCALE_FP16, 8, kRB>;
    case 4: return k_stream_single<XT, WAL_SCALE_FP24, 0, kRB>;
    case 5: return k_stream_single<XT, WAL_SCALE_FP24, 2, kRB>;
    case 6: return k_stream_single<XT, WAL_SCALE_FP24, 4, kRB>;
    default: return k_stream_single<XT, WAL_SCALE_FP24, 8, kRB>;
  }
}
// Streaming kernel of a class; NULL when the combination is not built
// (base-3 codes take bf16 activations only).
GroupedFn grouped_for(int x_dtype, uint32_t cls) {
  if (cls >= 8) return x_dtype == WAL_X_BF16 ? base3_grouped_kernel(cls) : nullptr;
  return x_dtype == WAL_X_BF16 ? grouped_kernel<WAL_X_BF16>(cls) : grouped_kernel<WAL_X_F32>(cls);
}
SingleFn single_for(int x_dtype, uint32_t cls) {
  if (cls >= 8) return x_dtype == WAL_X_BF16 ? base3_single_kernel(cls) : nullptr;
  return x_dtype == WAL_X_BF16 ? single_kernel<WAL_X_BF16>(cls) : single_kernel<WAL_X_F32>(cls);
}

// Workgroups of a streaming kernel that the current device holds at once.
int resident_blocks(const void* kernel, uint32_t* out) {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return WAL_ERR_DEVICE;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return WAL_ERR_DEVICE;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, kThreads, 0) != hipSuccess) return WAL_ERR_DEVICE;
  if (cus <= 0 || per <= 0) return WAL_ERR_DEVICE;
  *out = (uint32_t)(cus * per);
  return WAL_OK;
}

// Bytes one row of a matrix contributes to the stream (codes, sites, scales, U).
uint64_t row_bytes(const wal_info& f) {
  const uint64_t in = f.d.in, G = f.groups, sb = f.d.scale_fmt == WAL_SCALE_FP16 ? 2 : 3;
  const uint64_t codes = f.d.trit_fmt == WAL_TRIT_2BIT ? in / 4 : (in + 4) / 5;
  return codes + G * f.d.k + G * sb * (f.d.k ? 2 : 1) + (uint64_t)f.d.n_paths * ((f.d.rank + 7) / 8);
}

// Low-rank column chunks of a matrix in a grouped product (one partial sum of
// z per chunk: jobs stay short however wide the matrix).
uint32_t grouped_zc(const wal_info& f) { return (f.d.in + kZChunkCols - 1) / kZChunkCols; }

uint64_t count_zjobs(uint32_t n, const wal_info* infos) {
  uint64_t j = 0;
  for (uint32_t i = 0; i < n; ++i) {
    const uint32_t T = infos[i].d.n_paths * infos[i].d.rank;
    j += (uint64_t)(T + kZTerms - 1) / kZTerms * (T ? grouped_zc(infos[i]) : 0);
  }
  return j;
}

int check_blob_size(const wal_info* f) {
  if (f->total_bytes - f->off_codes >= (1ull << 32)) return WAL_ERR_UNSUPPORTED;
  return WAL_OK;
}

// Layout of a grouped plan: header | MatDev[n] | zjobs | per class:
// blockseg[grid + 1] | segs[matrices of the class + grid].
struct PlanShape {
  uint32_t n_classes;
  uint32_t cls[WAL_MAX_CLASSES], grid[WAL_MAX_CLASSES], mats[WAL_MAX_CLASSES];
  uint64_t rows[WAL_MAX_CLASSES];
  uint64_t off_descs, off_zjobs, off_blockseg[WAL_MAX_CLASSES], off_segs[WAL_MAX_CLASSES], bytes;
};

int plan_shape(uint32_t n, const wal_info* infos, uint32_t grid, int x_dtype, PlanShape* P) {
  std::memset(P, 0, sizeof(*P));
  uint64_t rows[kClasses] = {0};
  uint32_t mats[kClasses] = {0};
  for (uint32_t i = 0; i < n; ++i) {
    const uint32_t c = class_of(infos[i].d);
    rows[c] += infos[i].d.out;
    ++mats[c];
  }
  for (uint32_t c = 0; c < kClasses; ++c) {
    if (!mats[c]) continue;
    if (!grouped_for(x_dtype, c)) return WAL_ERR_UNSUPPORTED;
    uint32_t g = grid;
    if (!g) {
      uint32_t res = 0;
      int st = resident_blocks(reinterpret_cast<const void*>(grouped_for(x_dtype, c)), &res);
      if (st) return st;
      const uint64_t by_rows = (rows[c] + 15) / 16;
      g = (uint32_t)(by_rows < res ? by_rows : res);
      if (!g) g = 1;
    }
    const uint32_t k = P->n_classes++;
    P->cls[k] = c;
    P->grid[k] = g;
    P->mats[k] = mats[c];
    P->rows[k] = rows[c];
  }
  uint64_t off = up64(sizeof(PlanHeader), 64);
  P->off_descs = off;
  off += up64((uint64_t)n * sizeof(MatDev), 64);
  P->off_zjobs = off;
  off += up64(count_zjobs(n, infos) * 8, 64);   // (matrix, t0 << 16 | chunk) pairs
  for (uint32_t k = 0; k < P->n_classes; ++k) {
    P->off_blockseg[k] = off;
    off += up64(4ull * (P->grid[k] + 1), 64);
    P->off_segs[k] = off;
    off += up64(((uint64_t)P->mats[k] + P->grid[k] + P->rows[k] / seg_rows(P->cls[k]) + 1) * sizeof(Seg), 64);
  }
  P->bytes = off;
  return WAL_OK;
}

}  // namespace

extern "C" {

int wal_gemv(const wal_info* info, const void* W_dev, const void* x_dev, int x_dtype, float* y_dev,
             void* ws_dev, size_t ws_bytes, void* stream) {
  int st = check_info(info);
  if (st) return st;
  if (!W_dev || !x_dev || !y_dev) return WAL_ERR_ARG;
  if (x_dtype != WAL_X_F32 && x_dtype != WAL_X_BF16) return WAL_ERR_ARG;
  if (!aligned(W_dev, 256) || !aligned(x_dev, 16) || !aligned(y_dev, 4)) return WAL_ERR_ALIGN;
  const GemmShape S = gemm_shape(*info, 1);
  const uint32_t cls = class_of(info->d);
  const uint32_t npass = cls >= 8 ? (info->d.in + kPassBase3 - 1) / kPassBase3 : (info->d.in + kPass2bit - 1) / kPass2bit;
  // Matrices wider than one pass run their passes in separate workgroups
  // when the workspace holds the per-pass partial sums (it does at
  // wal_workspace_size(info, 1) bytes); a reduce adds them.
  const bool split = npass > 1 && ws_dev && ws_bytes >= S.bytes;
  const size_t need = split ? (size_t)S.bytes : info->d.n_paths ? (size_t)S.off_p : 0;   // z partials [chunks][terms]
  if (need && (!ws_dev || ws_bytes < need)) return ws_dev ? WAL_ERR_BUFFER : WAL_ERR_ARG;
  if (need && !aligned(ws_dev, 16)) return WAL_ERR_ALIGN;
  if (overlap(x_dev, (size_t)info->d.in * xelem(x_dtype), y_dev, (size_t)info->d.out * 4)) return WAL_ERR_ARG;
  if (need && (overlap(ws_dev, need, y_dev, (size_t)info->d.out * 4) ||
               overlap(ws_dev, need, x_dev, (size_t)info->d.in * xelem(x_dtype))))
    return WAL_ERR_ARG;
  if ((st = check_blob_size(info))) return st;
  if (!single_for(x_dtype, cls)) return WAL_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  MatDev d = make_dev(info, W_dev, x_dev, y_dev, static_cast<float*>(ws_dev), info->d.in, info->d.out, 1);
  d.zc = (info->d.in + kZSingleCols - 1) / kZSingleCols;   // at most S.zc partials
  if (d.terms) {
    const uint32_t g = (d.terms + kZTerms - 1) / kZTerms * d.zc;
    if (x_dtype == WAL_X_BF16) hipLaunchKernelGGL(k_z_chunks<WAL_X_BF16>, dim3(g), dim3(kThreads), 0, s, d);
    else hipLaunchKernelGGL(k_z_chunks<WAL_X_F32>, dim3(g), dim3(kThreads), 0, s, d);
    if ((st = launch_status())) return st;
  }
  uint32_t resident = 0;
  if ((st = resident_blocks(reinterpret_cast<const void*>(grouped_for(x_dtype, cls)), &resident))) return st;
  // rows per block: the (row, pass) work spread evenly over the blocks the
  // GPU holds at once
  const uint64_t units = (uint64_t)d.out * (split ? npass : 1);
  uint32_t rpb = (uint32_t)((units + resident - 1) / resident);
  const uint32_t min_rows = kWaves * kRB;   // one batch per wavefront
  if (rpb < min_rows) rpb = min_rows;
  rpb = (rpb + kRB - 1) / kRB * kRB;
  if (rpb > seg_rows(cls)) rpb = seg_rows(cls);
  const uint32_t nrb = (d.out + rpb - 1) / rpb;
  float* P = split ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws_dev) + S.off_p) : nullptr;
  hipLaunchKernelGGL(single_for(x_dtype, cls), dim3(nrb * (split ? npass : 1)), dim3(kThreads), 0, s, d, rpb, nrb, P);
  if ((st = launch_status()) || !split) return st;
  return launch_reduce_single(d, d.z, d.zc, P, npass, stream);
}

int wal_gemm_small(const wal_info* info, const void* W_dev, const void* X_dev, int x_dtype, uint32_t batch,
                   uint32_t ldx, float* Y_dev, uint32_t ldy, int mode, void* ws_dev, size_t ws_bytes,
                   void* stream) {
  int st = check_info(info);
  if (st) return st;
  if (batch == 0 || batch > WAL_MAX_BATCH) return WAL_ERR_ARG;
  if (mode < WAL_GEMM_AUTO || mode > WAL_GEMM_MFMA) return WAL_ERR_ARG;
  if (!W_dev || !X_dev || !Y_dev) return WAL_ERR_ARG;
  if (x_dtype != WAL_X_F32 && x_dtype != WAL_X_BF16) return WAL_ERR_ARG;
  if (ldx < info->d.in || ldy < info->d.out) return WAL_ERR_ARG;
  const size_t xe = xelem(x_dtype);
  if (!aligned(W_dev, 256) || !aligned(X_dev, 16) || !aligned(Y_dev, 4) || (ldx * xe) % 16) return WAL_ERR_ALIGN;
  size_t need = 0;
  if ((st = wal_workspace_size(info, batch, &need))) return st;
  if (!ws_dev || ws_bytes < need) return ws_dev ? WAL_ERR_BUFFER : WAL_ERR_ARG;
  if (!aligned(ws_dev, 16)) return WAL_ERR_ALIGN;
  const size_t xbytes = ((size_t)(batch - 1) * ldx + info->d.in) * xe;
  const size_t ybytes = ((size_t)(batch - 1) * ldy + info->d.out) * 4;
  if (xbytes >= (1ull << 31)) return WAL_ERR_SHAPE;   // X is addressed with 32-bit byte offsets
  if (overlap(X_dev, xbytes, Y_dev, ybytes) || overlap(ws_dev, need, Y_dev, ybytes) ||
      overlap(ws_dev, need, X_dev, xbytes))
    return WAL_ERR_ARG;
  if ((st = check_blob_size(info))) return st;
  // The batched kernels take bf16 activations and 2-bit codes; other inputs
  // run one batch-1 product per column.
  const bool batched = x_dtype == WAL_X_BF16 && info->d.trit_fmt == WAL_TRIT_2BIT;
  bool per_row = !batched;
  if (mode == WAL_GEMM_AUTO) {
    mode = batched && batch >= kGemmCrossover ? WAL_GEMM_MFMA : WAL_GEMM_VALU;
    per_row = per_row || batch == 1;
  }
  MatDev d = make_dev(info, W_dev, X_dev, Y_dev, static_cast<float*>(ws_dev), ldx, ldy, batch);
  if (mode == WAL_GEMM_MFMA) {
    if (!batched) return WAL_ERR_UNSUPPORTED;
    return launch_gemm_mfma(*info, d, batch, ws_dev, stream);
  }
  if (!per_row) return launch_gemm_valu(*info, d, batch, ws_dev, stream);
  for (uint32_t n = 0; n < batch; ++n) {
    const void* xn = static_cast<const uint8_t*>(X_dev) + (size_t)n * ldx * xe;
    if ((st = wal_gemv(info, W_dev, xn, x_dtype, Y_dev + (size_t)n * ldy, ws_dev, ws_bytes, stream))) return st;
  }
  return WAL_OK;
}

int wal_gemm_prefill(const wal_info* info, const void* W_dev, const void* X_dev, int x_dtype, uint32_t batch,
                     uint32_t ldx, float* Y_dev, uint32_t ldy, void* ws_dev, size_t ws_bytes, void* stream) {
  int st = check_info(info);
  if (st) return st;
  if (batch == 0 || batch > WAL_MAX_PREFILL_BATCH) return WAL_ERR_ARG;
  if (!W_dev || !X_dev || !Y_dev) return WAL_ERR_ARG;
  if (x_dtype != WAL_X_F32 && x_dtype != WAL_X_BF16) return WAL_ERR_ARG;
  if (ldx < info->d.in || ldy < info->d.out) return WAL_ERR_ARG;
  if (x_dtype != WAL_X_BF16 || info->d.trit_fmt != WAL_TRIT_2BIT) return WAL_ERR_UNSUPPORTED;
  if (!aligned(W_dev, 256) || !aligned(X_dev, 16) || !aligned(Y_dev, 4) || (ldx * 2u) % 16) return WAL_ERR_ALIGN;
  const size_t xbytes = ((size_t)(batch - 1) * ldx + info->d.in) * 2;
  const size_t ybytes = ((size_t)(batch - 1) * ldy + info->d.out) * 4;
  if (xbytes >= (1ull << 31)) return WAL_ERR_SHAPE;   // X is addressed with 32-bit byte offsets
  size_t need = 0;
  if ((st = wal_prefill_workspace_size(info, batch, &need))) return st;
  if (need && (!ws_dev || ws_bytes < need)) return ws_dev ? WAL_ERR_BUFFER : WAL_ERR_ARG;
  if (ws_dev && !aligned(ws_dev, 16)) return WAL_ERR_ALIGN;
  if (overlap(X_dev, xbytes, Y_dev, ybytes) || (need && (overlap(ws_dev, need, Y_dev, ybytes) ||
                                                         overlap(ws_dev, need, X_dev, xbytes))))
    return WAL_ERR_ARG;
  if ((st = check_blob_size(info))) return st;
  MatDev d = make_dev(info, W_dev, X_dev, Y_dev, static_cast<float*>(ws_dev), ldx, ldy, batch);
  return launch_gemm_prefill(*info, d, batch, ws_dev, stream);
}

int wal_grouped_plan_size(uint32_t n, const wal_info* infos, uint32_t grid, int x_dtype, size_t* plan_bytes,
                          size_t* ws_bytes) {
  if (!n || !infos || !plan_bytes || !ws_bytes) return WAL_ERR_ARG;
  if (x_dtype != WAL_X_F32 && x_dtype != WAL_X_BF16) return WAL_ERR_ARG;
  if (n > (1u << 24)) return WAL_ERR_ARG;
  uint64_t ws = 0;
  for (uint32_t i = 0; i < n; ++i) {
    int st = check_info(&infos[i]);
    if (st) return st;
    if ((st = check_blob_size(&infos[i]))) return st;
    const uint64_t T = (uint64_t)infos[i].d.n_paths * infos[i].d.rank;
    ws += T ? up64(4 * T * grouped_zc(infos[i]), 16) : 0;
  }
  PlanShape P;
  int st = plan_shape(n, infos, grid, x_dtype, &P);
  if (st) return st;
  *plan_bytes = (size_t)P.bytes;
  *ws_bytes = (size_t)up64(ws, 256);
  return WAL_OK;
}

int wal_grouped_plan(uint32_t n, const wal_info* infos, const void* const* W_dev, const void* const* x_dev,
                     int x_dtype, float* const* y_dev, void* ws_dev, size_t ws_bytes, uint32_t grid,
                     void* plan_host, size_t plan_bytes, wal_grouped_info* ginfo) {
  size_t need_plan = 0, need_ws = 0;
  int st = wal_grouped_plan_size(n, infos, grid, x_dtype, &need_plan, &need_ws);
  if (st) return st;
  if (!W_dev || !x_dev || !y_dev || !plan_host || !ginfo) return WAL_ERR_ARG;
  if (plan_bytes < need_plan) return WAL_ERR_BUFFER;
  if (need_ws && (!ws_dev || ws_bytes < need_ws)) return ws_dev ? WAL_ERR_BUFFER : WAL_ERR_ARG;
  if (need_ws && !aligned(ws_dev, 16)) return WAL_ERR_ALIGN;
  for (uint32_t i = 0; i < n; ++i) {
    if (!W_dev[i] || !x_dev[i] || !y_dev[i]) return WAL_ERR_ARG;
    if (!aligned(W_dev[i], 256) || !aligned(x_dev[i], 16) || !aligned(y_dev[i], 4)) return WAL_ERR_ALIGN;
    if (overlap(x_dev[i], (size_t)infos[i].d.in * xelem(x_dtype), y_dev[i], (size_t)infos[i].d.out * 4))
      return WAL_ERR_ARG;
  }
  PlanShape P;
  if ((st = plan_shape(n, infos, grid, x_dtype, &P))) return st;
  uint8_t* base = static_cast<uint8_t*>(plan_host);
  std::memset(base, 0, P.bytes);
  PlanHeader* h = reinterpret_cast<PlanHeader*>(base);
  MatDev* descs = reinterpret_cast<MatDev*>(base + P.off_descs);
  uint32_t* jobs = reinterpret_cast<uint32_t*>(base + P.off_zjobs);

  // descriptors and low-rank jobs
  uint64_t zoff = 0, j = 0;
  for (uint32_t i = 0; i < n; ++i) {
    const uint32_t T = infos[i].d.n_paths * infos[i].d.rank, zc = grouped_zc(infos[i]);
    float* z = T ? static_cast<float*>(ws_dev) + zoff / 4 : nullptr;
    descs[i] = make_dev(&infos[i], W_dev[i], x_dev[i], y_dev[i], z, infos[i].d.in, infos[i].d.out, 1);
    descs[i].zc = zc;   // z partials [zc][T]
    zoff += T ? up64(4ull * T * zc, 16) : 0;
    for (uint32_t cc = 0; T && cc < zc; ++cc)
      for (uint32_t t0 = 0; t0 < T; t0 += kZTerms) {
        jobs[2 * j] = i;
        jobs[2 * j + 1] = (t0 << 16) | cc;
        ++j;
      }
  }

  std::memset(ginfo, 0, sizeof(*ginfo));
  uint32_t nseg_total = 0, gmax = 0;
  for (uint32_t k = 0; k < P.n_classes; ++k) {
    // The class's matrices in order; their rows are split into grid ranges
    // of equal streamed bytes, one per workgroup.
    const uint32_t c = P.cls[k], G = P.grid[k];
    uint32_t* blockseg = reinterpret_cast<uint32_t*>(base + P.off_blockseg[k]);
    Seg* segs = reinterpret_cast<Seg*>(base + P.off_segs[k]);
    uint64_t total = 0;
    for (uint32_t i = 0; i < n; ++i)
      if (class_of(infos[i].d) == c) total += row_bytes(infos[i]) * infos[i].d.out;
    // boundary b: (matrix, row) where the b-th range starts; mat == n past the end
    auto boundary = [&](uint32_t b, uint32_t* mat, uint32_t* row) {
      const uint64_t pos = (uint64_t)((unsigned __int128)total * b / G);
      uint64_t acc = 0;
      for (uint32_t i = 0; i < n; ++i) {
        if (class_of(infos[i].d) != c) continue;
        const uint64_t rb = row_bytes(infos[i]), mb = rb * infos[i].d.out;
        if (pos < acc + mb) {
          const uint64_t r = (pos - acc + rb / 2) / rb;
          *mat = i;
          *row = (uint32_t)r;
          if (r >= infos[i].d.out) {   // rounds to the next matrix of the class
            uint32_t nx = i + 1;
            while (nx < n && class_of(infos[nx].d) != c) ++nx;
            *mat = nx;
            *row = 0;
          }
          return;
        }
        acc += mb;
      }
      *mat = n;
      *row = 0;
    };
    uint32_t nseg = 0, m0 = 0, r0 = 0;
    boundary(0, &m0, &r0);
    for (uint32_t b = 0; b < G; ++b) {
      blockseg[b] = nseg;
      uint32_t m1 = 0, r1 = 0;
      boundary(b + 1, &m1, &r1);
      for (uint32_t m = m0; m < n && m <= m1; ++m) {
        if (class_of(infos[m].d) != c) continue;
        const uint32_t rs = m == m0 ? r0 : 0;
        const uint32_t re = m == m1 ? r1 : infos[m].d.out;
        const uint32_t sr = seg_rows(c);
        for (uint32_t r = rs; r < re; r += sr) segs[nseg++] = Seg{m, r, re - r > sr ? r + sr : re, 0};
      }
      m0 = m1;
      r0 = r1;
    }
    blockseg[G] = nseg;
    ginfo->class_id[k] = c;
    ginfo->class_grid[k] = G;
    ginfo->class_blockseg[k] = P.off_blockseg[k];
    ginfo->class_segs[k] = P.off_segs[k];
    nseg_total += nseg;
    if (G > gmax) gmax = G;
  }

  h->magic = kPlanMagic;
  h->n = n;
  h->grid = gmax;
  h->n_segs = nseg_total;
  h->n_zjobs = (uint32_t)j;
  h->x_dtype = (uint32_t)x_dtype;
  h->trit_fmt = 0;
  h->reserved = P.n_classes;
  h->off_descs = P.off_descs;
  h->off_zjobs = P.off_zjobs;
  h->bytes = P.bytes;

  ginfo->n = n;
  ginfo->n_classes = P.n_classes;
  ginfo->n_segs = nseg_total;
  ginfo->n_zjobs = (uint32_t)j;
  ginfo->x_dtype = (uint32_t)x_dtype;
  ginfo->trit_fmt = 0;
  ginfo->rows_per_batch = kRB;
  ginfo->grid = gmax;
  ginfo->plan_bytes = P.bytes;
  ginfo->off_descs = P.off_descs;
  ginfo->off_zjobs = P.off_zjobs;
  uint64_t alg = 0;
  for (uint32_t i = 0; i < n; ++i) alg += infos[i].algorithmic_bytes;
  ginfo->algorithmic_bytes = alg;
  return WAL_OK;
}

int wal_gemv_grouped_phases(const wal_grouped_info* g, const void* plan_dev, int phases, void* stream) {
  if (!g || !plan_dev) return WAL_ERR_ARG;
  if (phases < 1 || phases > WAL_PHASE_ALL) return WAL_ERR_ARG;
  if (!aligned(plan_dev, 16)) return WAL_ERR_ALIGN;
  if (g->x_dtype > WAL_X_BF16 || !g->n) return WAL_ERR_ARG;
  if (g->rows_per_batch != (uint32_t)kRB || !g->n_classes || g->n_classes > WAL_MAX_CLASSES) return WAL_ERR_ARG;
  for (uint32_t k = 0; k < g->n_classes; ++k) {
    if (g->class_id[k] >= kClasses || !g->class_grid[k]) return WAL_ERR_ARG;
    if (!grouped_for((int)g->x_dtype, g->class_id[k])) return WAL_ERR_UNSUPPORTED;
    if (g->class_blockseg[k] >= g->plan_bytes || g->class_segs[k] >= g->plan_bytes) return WAL_ERR_ARG;
  }
  if (g->off_descs >= g->plan_bytes || (g->n_zjobs && g->off_zjobs >= g->plan_bytes)) return WAL_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* base = static_cast<const uint8_t*>(plan_dev);
  const MatDev* descs = reinterpret_cast<const MatDev*>(base + g->off_descs);
  const uint32_t* jobs = reinterpret_cast<const uint32_t*>(base + g->off_zjobs);
  int st;
  if ((phases & WAL_PHASE_LOWRANK) && g->n_zjobs) {
    if (g->x_dtype == WAL_X_BF16)
      hipLaunchKernelGGL(k_z_grouped<WAL_X_BF16>, dim3(g->n_zjobs), dim3(kThreads), 0, s, descs, jobs);
    else
      hipLaunchKernelGGL(k_z_grouped<WAL_X_F32>, dim3(g->n_zjobs), dim3(kThreads), 0, s, descs, jobs);
    if ((st = launch_status())) return st;
  }
  for (uint32_t k = 0; (phases & WAL_PHASE_STREAM) && k < g->n_classes; ++k) {
    const uint32_t* blockseg = reinterpret_cast<const uint32_t*>(base + g->class_blockseg[k]);
    const Seg* segs = reinterpret_cast<const Seg*>(base + g->class_segs[k]);
    hipLaunchKernelGGL(grouped_for((int)g->x_dtype, g->class_id[k]), dim3(g->class_grid[k]), dim3(kThreads), 0, s,
                       descs, blockseg, segs);
    if ((st = launch_status())) return st;
  }
  return WAL_OK;
}

int wal_gemv_grouped(const wal_grouped_info* g, const void* plan_dev, void* stream) {
  return wal_gemv_grouped_phases(g, plan_dev, WAL_PHASE_ALL, stream);
}

int wal_gemv_grouped_seq(uint32_t n, const wal_grouped_info* ginfos, const void* const* plans_dev, void* stream) {
  if (!n || !ginfos || !plans_dev) return WAL_ERR_ARG;
  for (uint32_t i = 0; i < n; ++i) {
    const int st = wal_gemv_grouped(&ginfos[i], plans_dev[i], stream);
    if (st) return st;
  }
  return WAL_OK;
}

}  // extern "C"

// The captured chain: the executable graph and the graph it came from.
struct wal_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

extern "C" {

int wal_graph_create(uint32_t n, const wal_grouped_info* ginfos, const void* const* plans_dev, wal_graph** out) {
  if (!n || !ginfos || !plans_dev || !out) return WAL_ERR_ARG;
  *out = nullptr;
  hipStream_t s = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return WAL_ERR_DEVICE;
  if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipStreamDestroy(s);
    return WAL_ERR_DEVICE;
  }
  const int st = wal_gemv_grouped_seq(n, ginfos, plans_dev, s);
  hipGraph_t graph = nullptr;
  const hipError_t ce = hipStreamEndCapture(s, &graph);
  (void)hipStreamDestroy(s);
  if (st || ce != hipSuccess || !graph) {
    if (graph) (void)hipGraphDestroy(graph);
    return st ? st : WAL_ERR_DEVICE;
  }
  hipGraphExec_t exec = nullptr;
  if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return WAL_ERR_DEVICE;
  }
  wal_graph* g = new (std::nothrow) wal_graph{graph, exec};
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return WAL_ERR_DEVICE;
  }
  *out = g;
  return WAL_OK;
}

int wal_graph_launch(const wal_graph* g, void* stream) {
  if (!g) return WAL_ERR_ARG;
  return hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)) == hipSuccess ? WAL_OK : WAL_ERR_DEVICE;
}

int wal_graph_destroy(wal_graph* g) {
  if (!g) return WAL_OK;
  const bool ok = hipGraphExecDestroy(g->exec) == hipSuccess && hipGraphDestroy(g->graph) == hipSuccess;
  delete g;
  return ok ? WAL_OK : WAL_ERR_DEVICE;
}

}  // extern "C"
