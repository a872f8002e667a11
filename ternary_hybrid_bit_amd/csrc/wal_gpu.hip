// gfx950 (CDNA4) kernels and the product entry points of libwal.
//
// Operator (WAL-Ternary-8B cards, "Модель пішімі" / "Representation"):
//     y = (alpha * T + beta * R) x + sum_p U_p diag(s_p) V_p^T x
// computed straight from the packed planes described in include/wal.h.
//
// Kernels:
//  * k_stream_*: one launch per product (per (scale format, k) class of a
//    grouped plan).  Its first workgroups compute the binary low-rank
//    reductions z_p[r] = s_p[r] * sum_j (-1)^{V bit} x_j as jobs of a few
//    terms over a column chunk (partial sums per chunk, in the workspace);
//    the others stream the packed planes and wait for those jobs only in
//    their epilogue (wal_device.h, fused launches).
//    A streaming workgroup owns a contiguous range of rows of one or more
//    matrices (for grouped products the host splits the total packed bytes
//    evenly over a grid that fits the GPU at once), or one pass of a row
//    block of a wide single product.  Inside a range, the 4 wavefronts take
//    batches of RB rows in turn:
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
//        each row's total lands in 64/RB lanes, one of which keeps it in LDS.
//        Matrices wider than one pass accumulate it pass by pass.
//      - epilogue: tables of signed z sums, one per path and U byte, turn the
//        low-rank term of a row into one LDS lookup per U byte; then y.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <hip/hip_fp16.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

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

  // The same columns from activations staged in LDS (element e on).
  static __device__ __forceinline__ void load_lds(const void* xs, uint32_t e, Raw& r) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xs) + e);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 v = src[q];
      r.w[4 * q] = v.x; r.w[4 * q + 1] = v.y; r.w[4 * q + 2] = v.z; r.w[4 * q + 3] = v.w;
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

  static __device__ __forceinline__ void load_lds(const void* xs, uint32_t e, Raw& r) {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(xs) + e);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float4 v = src[q];
      r.f[4 * q] = v.x; r.f[4 * q + 1] = v.y; r.f[4 * q + 2] = v.z; r.f[4 * q + 3] = v.w;
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
};

// Per-pass lane constants of the 2-bit stream.
struct Lane2 {
  __amdgpu_buffer_rsrc_t rw;  // the blob from the codes plane on
  uint32_t vc, vs, va, vb;    // lane offsets (from the codes plane) in row 0 of each plane
  uint32_t sc, ss, sa;        // row strides (bytes) of each plane
  const float* tb;            // the lane's group in the site table
};

// One pass of one segment.  The workgroup-wide set-up of the pass (the site
// table, behind barriers) runs after each wave has issued the loads of its
// first batch and of its x columns, so the set-up overlaps the memory
// latency instead of adding to it.  Every wave reaches both barriers.  The
// low-rank term is added after the segment's last pass (store_segment).
template <int XT, int SF, int K, int RB, bool ROT>
__device__ __forceinline__ void stream_rows_2bit(const MatDev& d, uint32_t row0, uint32_t row1, uint32_t pass,
                                                 bool first, StreamSmem& sm) {
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
    const uint32_t row = row0 + yi;
    if ((lane & (LPR - 1)) == 0 && row < row1)
      sm.ybuf[yi] = v;
  };

  // Set-up loads first: the lane's x and the x of its share of the site
  // table (L2 hits).  Vector memory loads complete in order, so waiting for
  // these after the first batch's loads (HBM) are issued does not wait for
  // the batch.
  // A rotated product (ROT) instead has the workgroup rotate the whole
  // pass's 32 groups (RotPass); the pass then goes through LDS twice, as
  // compact activations that each lane reads its columns from, and as the
  // table.
  const __amdgpu_buffer_rsrc_t rx = x_rsrc<XT>(d.x, d.in);
  RotPass<XT, 32> rp;
  typename XLane<XT>::Raw xr;
  TableX<XT> tx;
  if constexpr (ROT) {
    rp.load(rx, pass * kPass2bit);
  } else {
    XLane<XT>::load_raw(rx, pass * kPass2bit + 64 * lane, xr);
    if constexpr (K > 0) tx.load(rx, pass * kPass2bit);
  }

  // Two batches in registers: while one is reduced, the next is in flight
  // (three resident workgroups per CU keep three wavefronts per SIMD, six
  // batches, in flight).
  Batch<RB> B0 = load_batch(b);
  if constexpr (ROT) rp.compute();

  __syncthreads();   // readers of the previous table are done
  if constexpr (ROT) {
    rp.store_x(sm.tbl);
    __syncthreads();
    XLane<XT>::load_lds(sm.tbl, 64 * lane, xr);
    if constexpr (K > 0) {
      __syncthreads();   // every lane has its columns
      rp.store_tbl(sm.tbl, 32);
    }
  } else if constexpr (K > 0) {
    tx.store(sm.tbl);
  }
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

// One segment (rows row0..row1-1 of one matrix) of a workgroup, pass by pass,
// then its store (store_segment: the low-rank term, or with P one pass's
// partial sums and the reduce of a completed row block).  SF and K are the
// matrix's scale format and sites per group: every (scale format, k) class
// has kernels of its own, so the registers of the hot fp16 / k = 8 loop are
// not set by the heavier fp24 loads.
// With count (the workgroup's last segment) the store may count the
// workgroup finished; returns whether it did.
template <int XT, int SF, int K, int RB, class ZJ, bool ROT>
__device__ __forceinline__ bool run_segment_2bit(const MatDev& d, uint32_t row0, uint32_t row1, StreamSmem& sm,
                                                 const Fuse& f, float* P = nullptr, uint32_t split_pass = 0,
                                                 uint32_t* cnt = nullptr, bool count = false) {
  const uint32_t npass = (d.in + kPass2bit - 1) / kPass2bit;
  const bool split = P != nullptr;
  const uint32_t p0 = split ? split_pass : 0, p1 = split ? split_pass + 1 : npass;
  for (uint32_t pass = p0; pass < p1; ++pass)
    stream_rows_2bit<XT, SF, K, RB, ROT>(d, row0, row1, pass, pass == p0, sm);
  return store_segment<XT, ZJ, ROT>(d, row0, row1, SegEnd{sm.tbl, sm.z, sm.ybuf}, f, P, split_pass, npass, cnt,
                                    count);
}

// Three workgroups per CU (the LDS of a workgroup allows it) when the class's
// registers fit three wavefronts per SIMD without spilling; the fp32 and the
// fp24 / k = 8 loops need more registers and run two.  Kernels that rotate x
// hold the rotation's operands while their first batch is in flight and run
// two (no spills).
constexpr int stream_waves_per_simd(int XT, int SF, int K, bool ROT) {
  return ROT ? 2 : XT == WAL_X_BF16 && !(SF == WAL_SCALE_FP24 && K == 8) ? 3 : 1;
}

// Low-rank job of a fused launch or of the grouped pre-pass: terms t0 ..
// t0 + terms - 1 of matrix m over columns [4096 cc, 4096 cc + 4096) into its
// partials z[cc][t] (jobs[2 j] = m, jobs[2 j + 1] = t0 << 16 | cc).
template <int XT, bool ROT>
__device__ __forceinline__ void grouped_z_job(const MatDev* __restrict__ descs, const uint32_t* __restrict__ jobs,
                                              uint32_t j, uint32_t terms, const uint32_t* epoch, void* xs) {
  const uint32_t m = jobs[2 * j], tc = jobs[2 * j + 1];
  const MatDev& d = descs[m];
  const uint32_t t0 = tc >> 16, cc = tc & 0xFFFFu;
  const uint32_t c0 = cc * kZChunkCols, c1 = min(d.in, c0 + kZChunkCols);
  z_job<XT, ZJobsGrouped, kZOutTagged, ROT>(d, terms, t0, reinterpret_cast<uint64_t*>(d.z) + (size_t)cc * d.terms, c0, c1,
                                      epoch, xs);
}

// Grouped products: workgroup t = blockIdx.x computes low-rank job t when
// t < f.nz, else streams the segments of block t - f.nz.
template <int XT, int SF, int K, int RB, bool ROT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(stream_waves_per_simd(XT, SF, K, ROT))))
void k_stream_grouped(const MatDev* __restrict__ descs, const uint32_t* __restrict__ blockseg,
                      const Seg* __restrict__ segs, const uint32_t* __restrict__ jobs, Fuse f) {
  __shared__ StreamSmem sm;
  const uint32_t t = blockIdx.x;
  bool counted = false;
  if (t < f.nz) {
    grouped_z_job<XT, ROT>(descs, jobs, t, zjob_terms<ZJobsGrouped>(f), epoch_of(f), sm.tbl);
  } else {
    const uint32_t b = t - f.nz;
    const uint32_t s0 = blockseg[b], s1 = blockseg[b + 1];
    for (uint32_t s = s0; s < s1; ++s) {
      const Seg sg = segs[s];
      const MatDev& d = descs[sg.mat];
      if (sg.pass1)
        counted = run_segment_2bit<XT, SF, K, RB, ZJobsGrouped, ROT>(d, sg.row0, sg.row1, sm, f, d.P, sg.pass1 - 1,
                                                                     f.sync + d.cnt_off, s + 1 == s1);
      else
        counted = run_segment_2bit<XT, SF, K, RB, ZJobsGrouped, ROT>(d, sg.row0, sg.row1, sm, f, nullptr, 0, nullptr,
                                                                     s + 1 == s1);
    }
  }
  if (!counted) finish_launch(f);
}

// Single products: workgroup t = blockIdx.x < f.nz computes the low-rank
// partials of terms kZTerms tc .. kZTerms tc + kZTerms - 1 over columns
// [8192 cc, 8192 cc + 8192) into d.z[cc][t] (t = cc tcs + tc); the others
// stream.  Without P, block b takes rows [b rpb, b rpb + rpb) over every
// pass; with P, block b takes pass b / nrb of row block b % nrb (rpb a
// multiple of 16; cnt: the arrival counters, one per 16 rows).
template <int XT, int SF, int K, int RB, bool ROT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(stream_waves_per_simd(XT, SF, K, ROT))))
void k_stream_single(MatDev d, uint32_t rows_per_block, uint32_t nrb, float* P, uint32_t* cnt, Fuse f) {
  __shared__ StreamSmem sm;
  const uint32_t t = blockIdx.x;
  bool counted = false;
  if (t < f.nz) {
    const uint32_t tcs = (d.terms + kZTerms - 1) / kZTerms, tc = t % tcs, cc = t / tcs;
    const uint32_t c0 = cc * kZSingleCols, c1 = min(d.in, c0 + kZSingleCols);
    z_chunk_rot<XT, (int)kZTerms, kZOutTagged, ROT>(d, tc * kZTerms, reinterpret_cast<uint64_t*>(d.z) + (size_t)cc * d.terms,
                                               c0, c1, epoch_of(f), sm.tbl);
  } else {
    const uint32_t b = t - f.nz;
    const uint32_t rb = P ? b % nrb : b;
    const uint32_t r0 = rb * rows_per_block;
    const uint32_t r1 = min(d.out, r0 + rows_per_block);
    if (r0 < r1)
      counted = run_segment_2bit<XT, SF, K, RB, ZJobsSingle, ROT>(d, r0, r1, sm, f, P, P ? b / nrb : 0u, cnt, true);
  }
  if (!counted) finish_launch(f);
}

// The grouped low-rank pre-pass as a launch of its own (the phase API).
template <int XT, bool ROT>
__global__ __launch_bounds__(kThreads) void k_z_grouped(const MatDev* __restrict__ descs,
                                                        const uint32_t* __restrict__ jobs, uint32_t terms) {
  __shared__ float xs[ROT ? kZChunkCols : 1];   // a rotated chunk
  grouped_z_job<XT, ROT>(descs, jobs, blockIdx.x, terms, nullptr, xs);
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

template <int XT, bool ROT>
GroupedFn grouped_kernel(uint32_t cls) {
  switch (cls) {
    case 0: return k_stream_grouped<XT, WAL_SCALE_FP16, 0, kRB, ROT>;
    case 1: return k_stream_grouped<XT, WAL_SCALE_FP16, 2, kRB, ROT>;
    case 2: return k_stream_grouped<XT, WAL_SCALE_FP16, 4, kRB, ROT>;
    case 3: return k_stream_grouped<XT, WAL_SCALE_FP16, 8, kRB, ROT>;
    case 4: return k_stream_grouped<XT, WAL_SCALE_FP24, 0, kRB, ROT>;
    case 5: return k_stream_grouped<XT, WAL_SCALE_FP24, 2, kRB, ROT>;
    case 6: return k_stream_grouped<XT, WAL_SCALE_FP24, 4, kRB, ROT>;
    default: return k_stream_grouped<XT, WAL_SCALE_FP24, 8, kRB, ROT>;
  }
}
template <int XT, bool ROT>
SingleFn single_kernel(uint32_t cls) {
  switch (cls) {
    case 0: return k_stream_single<XT, WAL_SCALE_FP16, 0, kRB, ROT>;
    case 1: return k_stream_single<XT, WAL_SCALE_FP16, 2, kRB, ROT>;
    case 2: return k_stream_single<XT, WAL_SCALE_FP16, 4, kRB, ROT>;
    case 3: return k_stream_single<XT, WAL_SCALE_FP16, 8, kRB, ROT>;
    case 4: return k_stream_single<XT, WAL_SCALE_FP24, 0, kRB, ROT>;
    case 5: return k_stream_single<XT, WAL_SCALE_FP24, 2, kRB, ROT>;
    case 6: return k_stream_single<XT, WAL_SCALE_FP24, 4, kRB, ROT>;
    default: return k_stream_single<XT, WAL_SCALE_FP24, 8, kRB, ROT>;
  }
}
// Streaming kernel of a class for activations of type x_dtype (with the
// rotation flag: the kernels that rotate x); NULL when the combination is
// not built (base-3 codes take bf16 activations only).
GroupedFn grouped_for(int x_dtype, uint32_t cls) {
  const bool rot = (x_dtype & WAL_X_ROT_H128) != 0;
  const int xt = x_dtype & ~WAL_X_ROT_H128;
  if (cls >= 8) return xt == WAL_X_BF16 ? base3_grouped_kernel(cls, rot) : nullptr;
  if (xt == WAL_X_BF16) return rot ? grouped_kernel<WAL_X_BF16, true>(cls) : grouped_kernel<WAL_X_BF16, false>(cls);
  return rot ? grouped_kernel<WAL_X_F32, true>(cls) : grouped_kernel<WAL_X_F32, false>(cls);
}
SingleFn single_for(int x_dtype, uint32_t cls) {
  const bool rot = (x_dtype & WAL_X_ROT_H128) != 0;
  const int xt = x_dtype & ~WAL_X_ROT_H128;
  if (cls >= 8) return xt == WAL_X_BF16 ? base3_single_kernel(cls, rot) : nullptr;
  if (xt == WAL_X_BF16) return rot ? single_kernel<WAL_X_BF16, true>(cls) : single_kernel<WAL_X_BF16, false>(cls);
  return rot ? single_kernel<WAL_X_F32, true>(cls) : single_kernel<WAL_X_F32, false>(cls);
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

// Grouped plans whose ranges hold at most this many streamed bytes snap
// range boundaries to matrix starts (within half a range).
constexpr uint64_t kSnapShareBytes = 256 << 10;

// Passes of a matrix (4096 columns, 5120 for base-3 codes) and the bytes a
// row contributes to pass p (its share of the row's bytes by width).
uint32_t mat_passes(const wal_info& f) {
  const uint32_t w = f.d.trit_fmt == WAL_TRIT_2BIT ? kPass2bit : kPassBase3;
  return (f.d.in + w - 1) / w;
}
uint64_t pass_row_bytes(const wal_info& f, uint32_t p) {
  const uint32_t w = f.d.trit_fmt == WAL_TRIT_2BIT ? kPass2bit : kPassBase3;
  const uint64_t pw = std::min<uint64_t>(w, f.d.in - (uint64_t)p * w);
  return std::max<uint64_t>(1, (row_bytes(f) * pw + f.d.in / 2) / f.d.in);
}

// Low-rank column chunks of a matrix in a grouped product (one partial sum of
// z per chunk: jobs stay short however wide the matrix).
uint32_t grouped_zc(const wal_info& f) { return (f.d.in + kZChunkCols - 1) / kZChunkCols; }

uint64_t count_zjobs(uint32_t n, const wal_info* infos, uint32_t terms) {
  uint64_t j = 0;
  for (uint32_t i = 0; i < n; ++i) {
    const uint32_t T = infos[i].d.n_paths * infos[i].d.rank;
    j += (uint64_t)(T + terms - 1) / terms * (T ? grouped_zc(infos[i]) : 0);
  }
  return j;
}

// Terms per low-rank job of a grouped plan.
uint32_t plan_zterms(uint32_t n, const wal_info* infos) {
  return count_zjobs(n, infos, kZTermsFew) <= kZJobsFewMax ? kZTermsFew : kZTermsMany;
}

int check_blob_size(const wal_info* f) {
  if (f->total_bytes - f->off_codes >= (1ull << 32)) return WAL_ERR_UNSUPPORTED;
  return WAL_OK;
}

// Layout of a grouped plan: header | MatDev[n] | zjobs | per class:
// blockseg[grid + 1] | segs[entries of the class + grid + ...].  Its
// workspace: the zero region (synchronisation words, then the arrival
// counters of split matrices, one u32 per 16 rows) when the plan has
// low-rank paths or split matrices, the low-rank partials, the partial sums
// of split matrices.
//
// A class whose 16-row groups are fewer than its workgroups splits its
// matrices of several passes into one entry per pass (workgroups then take
// rows of one pass, cut at multiples of 16 rows); other matrices are one
// entry over all passes.  The class's entries, in matrix order, are split
// into grid ranges of equal streamed bytes.
struct PlanShape {
  uint32_t n_classes, zterms;
  uint32_t cls[WAL_MAX_CLASSES], grid[WAL_MAX_CLASSES], entries[WAL_MAX_CLASSES];
  uint32_t kof[kClasses];   // launch index of a class id
  bool split[WAL_MAX_CLASSES];
  uint64_t rows[WAL_MAX_CLASSES];   // rows of the class's entries
  uint64_t counters;                // arrival counters of split matrices
  uint64_t off_descs, off_zjobs, off_blockseg[WAL_MAX_CLASSES], off_segs[WAL_MAX_CLASSES], bytes;
};
bool mat_split(const PlanShape& P, const wal_info& f) {
  return P.split[P.kof[class_of(f.d)]] && mat_passes(f) > 1;
}

// Whether a grouped plan's launches coordinate through the workspace's
// synchronisation words (low-rank jobs or split matrices).
bool plan_syncs(uint32_t n, const wal_info* infos, const PlanShape& P) {
  for (uint32_t i = 0; i < n; ++i)
    if (infos[i].d.n_paths || mat_split(P, infos[i])) return true;
  return false;
}

// Workspace of a grouped plan: the zero region (when the plan syncs), each
// matrix's tagged low-rank partials [zc][terms] (8 bytes each), then each
// split matrix's per-pass partial sums [passes][out]; the byte offsets of
// the partials per matrix (when zoff / poff are given) and the total.
uint64_t grouped_ws_bytes(uint32_t n, const wal_info* infos, const PlanShape& P, uint64_t* zoff, uint64_t* poff) {
  uint64_t off = plan_syncs(n, infos, P) ? kWsZeroBytes : 0;
  for (uint32_t i = 0; i < n; ++i) {
    const uint64_t T = (uint64_t)infos[i].d.n_paths * infos[i].d.rank;
    if (zoff) zoff[i] = off;
    off += T ? up64(8 * T * grouped_zc(infos[i]), 16) : 0;
  }
  off = up64(off, 256);
  for (uint32_t i = 0; i < n; ++i) {
    if (poff) poff[i] = off;
    if (mat_split(P, infos[i])) off += up64(4ull * mat_passes(infos[i]) * infos[i].d.out, 256);
  }
  return up64(off, 256);
}

static_assert(kSyncBytes == WAL_SYNC_BYTES && kSyncFallback == WAL_SYNC_FALLBACK_WORD,
              "synchronisation words as documented");
static_assert(kMaxRowBlocks == WAL_MAX_ROW_BLOCKS && kWsZeroBytes == WAL_WS_ZERO_BYTES && kWsZeroBytes % 256 == 0,
              "workspace zero region as documented");

int plan_shape(uint32_t n, const wal_info* infos, uint32_t grid, int x_dtype, PlanShape* P) {
  std::memset(P, 0, sizeof(*P));
  P->zterms = plan_zterms(n, infos);
  const uint64_t nzj = count_zjobs(n, infos, P->zterms);
  uint64_t groups[kClasses] = {0}, groups_split[kClasses] = {0};   // 16-row groups, and by pass
  uint32_t mats[kClasses] = {0};
  for (uint32_t i = 0; i < n; ++i) {
    const uint32_t c = class_of(infos[i].d), g16 = (infos[i].d.out + 15) / 16;
    groups[c] += g16;
    groups_split[c] += (uint64_t)g16 * mat_passes(infos[i]);
    ++mats[c];
  }
  for (uint32_t c = 0; c < kClasses; ++c) {
    if (!mats[c]) continue;
    if (!grouped_for(x_dtype, c)) return WAL_ERR_UNSUPPORTED;
    uint32_t g = grid, res = 0;
    if (!g) {
      int st = resident_blocks(reinterpret_cast<const void*>(grouped_for(x_dtype, c)), &res);
      if (st) return st;
      // the first launch also runs the low-rank jobs in workgroups of its
      // own: when they are few, its streaming workgroups leave them their
      // slots (many jobs belong to a large plan, whose long streaming
      // workgroups would leave those slots idle after the jobs end)
      if (P->n_classes == 0 && nzj <= res / 8) res -= (uint32_t)nzj;
    }
    // split when the class has fewer 16-row groups than workgroups and the
    // arrival counters of every split class fit the workspace's
    // kMaxRowBlocks words
    bool split = groups[c] < (g ? g : res) && groups_split[c] > groups[c];
    if (split) {
      uint64_t need = 0;
      for (uint32_t i = 0; i < n; ++i)
        if (class_of(infos[i].d) == c && mat_passes(infos[i]) > 1) need += (infos[i].d.out + 15) / 16;
      split = P->counters + need <= kMaxRowBlocks;
      if (split) P->counters += need;
    }
    if (!g) g = (uint32_t)std::max<uint64_t>(1, std::min<uint64_t>(split ? groups_split[c] : groups[c], res));
    const uint32_t k = P->n_classes++;
    P->cls[k] = c;
    P->kof[c] = k;
    P->grid[k] = g;
    P->split[k] = split;
  }
  for (uint32_t i = 0; i < n; ++i) {
    const uint32_t k = P->kof[class_of(infos[i].d)];
    const bool sp = mat_split(*P, infos[i]);
    const uint32_t e = sp ? mat_passes(infos[i]) : 1;
    P->entries[k] += e;
    P->rows[k] += (uint64_t)e * infos[i].d.out;
  }
  uint64_t off = up64(sizeof(PlanHeader), 64);
  P->off_descs = off;
  off += up64((uint64_t)n * sizeof(MatDev), 64);
  P->off_zjobs = off;
  off += up64(nzj * 8, 64);   // (matrix, t0 << 16 | chunk) pairs
  for (uint32_t k = 0; k < P->n_classes; ++k) {
    P->off_blockseg[k] = off;
    off += up64(4ull * (P->grid[k] + 1), 64);
    P->off_segs[k] = off;
    off += up64(((uint64_t)P->entries[k] + P->grid[k] + P->rows[k] / seg_rows(P->cls[k]) + 1) * sizeof(Seg), 64);
  }
  P->bytes = off;
  return WAL_OK;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free product (wal_gemv_noalloc): the workspace of
// wal_gemv (low-rank partials, and per-pass partial sums of a wide matrix) in
// a file-scope device array.  Each GPU the library runs on holds its own copy
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host it names a stand-in, not device memory): the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current.
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
static_assert(kScratchBytes == WAL_NOALLOC_SCRATCH_BYTES, "scratch size as declared in wal.h");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return WAL_ERR_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return WAL_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WAL_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return WAL_OK;
}

}  // namespace

extern "C" {

int wal_gemv(const wal_info* info, const void* W_dev, const void* x_dev, int x_dtype_flags, float* y_dev,
             void* ws_dev, size_t ws_bytes, void* stream) {
  int st = check_info(info);
  if (st) return st;
  if (!W_dev || !x_dev || !y_dev) return WAL_ERR_ARG;
  if (x_dtype_flags & ~(WAL_X_BF16 | WAL_X_ROT_H128)) return WAL_ERR_ARG;
  const int x_dtype = x_dtype_flags & ~WAL_X_ROT_H128;   // element type
  if (!aligned(W_dev, 256) || !aligned(x_dev, 16) || !aligned(y_dev, 4)) return WAL_ERR_ALIGN;
  const GemmShape S = gemm_shape(*info, 1);
  const uint32_t cls = class_of(info->d);
  const uint32_t npass = cls >= 8 ? (info->d.in + kPassBase3 - 1) / kPassBase3 : (info->d.in + kPass2bit - 1) / kPass2bit;
  // Matrices wider than one pass run their passes in separate workgroups
  // when the workspace holds the per-pass partial sums (it does at
  // wal_workspace_size(info, 1) bytes); the workgroup that completes a row
  // block adds them.  The workspace: synchronisation words, arrival
  // counters, low-rank partials [chunks][terms], partial sums.
  // A split product counts arrivals per 16 rows: at most kMaxRowBlocks
  // counters.
  const uint32_t out = info->d.out;
  const bool split = npass > 1 && ws_dev && ws_bytes >= S.bytes && (out + 15) / 16 <= kMaxRowBlocks;
  const size_t need = split ? (size_t)S.bytes : info->d.n_paths ? (size_t)S.off_p : 0;
  if (need && (!ws_dev || ws_bytes < need)) return ws_dev ? WAL_ERR_BUFFER : WAL_ERR_ARG;
  if (need && !aligned(ws_dev, 16)) return WAL_ERR_ALIGN;
  if (overlap(x_dev, (size_t)info->d.in * xelem(x_dtype), y_dev, (size_t)info->d.out * 4)) return WAL_ERR_ARG;
  if (need && (overlap(ws_dev, need, y_dev, (size_t)info->d.out * 4) ||
               overlap(ws_dev, need, x_dev, (size_t)info->d.in * xelem(x_dtype))))
    return WAL_ERR_ARG;
  if ((st = check_blob_size(info))) return st;
  if (!single_for(x_dtype_flags, cls)) return WAL_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(ws_dev);
  MatDev d = make_dev(info, W_dev, x_dev, y_dev, need ? reinterpret_cast<float*>(ws + S.off_z) : nullptr,
                      info->d.in, info->d.out, 1);
  d.zc = (info->d.in + kZSingleCols - 1) / kZSingleCols;   // at most S.zc partials
  uint32_t resident = 0;
  if ((st = resident_blocks(reinterpret_cast<const void*>(single_for(x_dtype_flags, cls)), &resident))) return st;
  // One launch: its first nz workgroups compute the low-rank partials, which
  // the others read only when they store their rows.
  const uint32_t nz = d.terms ? (d.terms + kZTerms - 1) / kZTerms * d.zc : 0;
  // rows per block: the (row, pass) work spread evenly over the blocks the
  // GPU holds at once besides the low-rank jobs
  const uint32_t slots = nz <= resident / 8 ? resident - nz : resident;
  const uint64_t units = (uint64_t)out * (split ? npass : 1);
  uint32_t rpb = (uint32_t)((units + slots - 1) / slots);
  rpb = std::max(rpb, kWaves * kRB);   // one batch per wavefront
  const uint32_t unit = split ? 16u : (uint32_t)kRB;   // split row blocks start at multiples of 16
  rpb = std::min((rpb + unit - 1) / unit * unit, seg_rows(cls));
  const uint32_t nrb = (out + rpb - 1) / rpb;
  float* P = split ? reinterpret_cast<float*>(ws + S.off_p) : nullptr;
  uint32_t* cnt = split ? reinterpret_cast<uint32_t*>(ws + S.off_cnt) : nullptr;
  const uint32_t grid = nz + nrb * (split ? npass : 1);
  Fuse f{};
  if (need) f = Fuse{reinterpret_cast<uint32_t*>(ws), 0u, nz, nz ? 1u : 0u, grid, 1u, kZTerms};
  hipLaunchKernelGGL(single_for(x_dtype_flags, cls), dim3(grid), dim3(kThreads), 0, s, d, rpb, nrb, P, cnt, f);
  return launch_status();
}

int wal_gemv_noalloc(const wal_info* info, const void* W_dev, const void* x_dev, int x_dtype, float* y_dev,
                     void* stream) {
  int st = check_info(info);
  if (st) return st;
  // The low-rank partials must fit; the per-pass partial sums of a wide
  // matrix are used when they fit too (else its passes run in sequence
  // inside each workgroup, as wal_gemv does with a short workspace).
  const GemmShape S = gemm_shape(*info, 1);
  if (info->d.n_paths && S.off_p > kScratchBytes) return WAL_ERR_BUFFER;
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return wal_gemv(info, W_dev, x_dev, x_dtype, y_dev, ws, kScratchBytes, stream);
}

int wal_gemm_small(const wal_info* info, const void* W_dev, const void* X_dev, int x_dtype, uint32_t batch,
                   uint32_t ldx, float* Y_dev, uint32_t ldy, int mode, void* ws_dev, size_t ws_bytes,
                   void* stream) {
  int st = check_info(info);
  if (st) return st;
  if (batch == 0 || batch > WAL_MAX_BATCH) return WAL_ERR_ARG;
  if (mode < WAL_GEMM_AUTO || mode > WAL_GEMM_MFMA) return WAL_ERR_ARG;
  if (!W_dev || !X_dev || !Y_dev) return WAL_ERR_ARG;
  if (x_dtype == (WAL_X_F32 | WAL_X_ROT_H128) || x_dtype == (WAL_X_BF16 | WAL_X_ROT_H128))
    return WAL_ERR_UNSUPPORTED;   // rotate X first (wal_rotate_h128)
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
  if (x_dtype == (WAL_X_F32 | WAL_X_ROT_H128) || x_dtype == (WAL_X_BF16 | WAL_X_ROT_H128))
    return WAL_ERR_UNSUPPORTED;   // rotate X first (wal_rotate_h128)
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

int wal_grouped_plan_size(uint32_t n, const wal_info* infos, uint32_t grid, int x_dtype_flags, size_t* plan_bytes,
                          size_t* ws_bytes) {
  if (!n || !infos || !plan_bytes || !ws_bytes) return WAL_ERR_ARG;
  if (x_dtype_flags & ~(WAL_X_BF16 | WAL_X_ROT_H128)) return WAL_ERR_ARG;
  if (n > (1u << 24)) return WAL_ERR_ARG;
  for (uint32_t i = 0; i < n; ++i) {
    int st = check_info(&infos[i]);
    if (st) return st;
    if ((st = check_blob_size(&infos[i]))) return st;
  }
  PlanShape P;
  int st = plan_shape(n, infos, grid, x_dtype_flags, &P);
  if (st) return st;
  *plan_bytes = (size_t)P.bytes;
  *ws_bytes = (size_t)grouped_ws_bytes(n, infos, P, nullptr, nullptr);
  return WAL_OK;
}

int wal_grouped_plan(uint32_t n, const wal_info* infos, const void* const* W_dev, const void* const* x_dev,
                     int x_dtype_flags, float* const* y_dev, void* ws_dev, size_t ws_bytes, uint32_t grid,
                     void* plan_host, size_t plan_bytes, wal_grouped_info* ginfo) {
  size_t need_plan = 0, need_ws = 0;
  int st = wal_grouped_plan_size(n, infos, grid, x_dtype_flags, &need_plan, &need_ws);
  if (st) return st;
  const int x_dtype = x_dtype_flags & ~WAL_X_ROT_H128;   // element type
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
  if ((st = plan_shape(n, infos, grid, x_dtype_flags, &P))) return st;
  uint8_t* base = static_cast<uint8_t*>(plan_host);
  std::memset(base, 0, P.bytes);
  PlanHeader* h = reinterpret_cast<PlanHeader*>(base);
  MatDev* descs = reinterpret_cast<MatDev*>(base + P.off_descs);
  uint32_t* jobs = reinterpret_cast<uint32_t*>(base + P.off_zjobs);

  // descriptors and low-rank jobs
  std::vector<uint64_t> zoff(n), poff(n);
  grouped_ws_bytes(n, infos, P, zoff.data(), poff.data());
  uint8_t* wsb = static_cast<uint8_t*>(ws_dev);
  uint64_t j = 0, cnt = kSyncBytes / 4;
  for (uint32_t i = 0; i < n; ++i) {
    const uint32_t T = infos[i].d.n_paths * infos[i].d.rank, zc = grouped_zc(infos[i]);
    float* z = T ? reinterpret_cast<float*>(wsb + zoff[i]) : nullptr;
    descs[i] = make_dev(&infos[i], W_dev[i], x_dev[i], y_dev[i], z, infos[i].d.in, infos[i].d.out, 1);
    descs[i].zc = zc;   // z partials [zc][T]
    if (mat_split(P, infos[i])) {
      descs[i].P = reinterpret_cast<float*>(wsb + poff[i]);
      descs[i].cnt_off = (uint32_t)cnt;
      cnt += (infos[i].d.out + 15) / 16;
    }
    for (uint32_t cc = 0; T && cc < zc; ++cc)
      for (uint32_t t0 = 0; t0 < T; t0 += P.zterms) {
        jobs[2 * j] = i;
        jobs[2 * j + 1] = (t0 << 16) | cc;
        ++j;
      }
  }

  std::memset(ginfo, 0, sizeof(*ginfo));
  uint32_t nseg_total = 0, gmax = 0;
  struct Entry {
    uint32_t mat, pass1, out;
    uint64_t rb;   // streamed bytes per row
  };
  std::vector<Entry> ent;
  for (uint32_t k = 0; k < P.n_classes; ++k) {
    // The class's entries in order; their rows are split into grid ranges of
    // equal streamed bytes, one per workgroup (at multiples of 16 rows in a
    // split entry, whose row groups count arrivals).
    const uint32_t c = P.cls[k], G = P.grid[k];
    uint32_t* blockseg = reinterpret_cast<uint32_t*>(base + P.off_blockseg[k]);
    Seg* segs = reinterpret_cast<Seg*>(base + P.off_segs[k]);
    ent.clear();
    uint64_t total = 0;
    for (uint32_t i = 0; i < n; ++i) {
      if (class_of(infos[i].d) != c) continue;
      if (mat_split(P, infos[i])) {
        for (uint32_t p = 0; p < mat_passes(infos[i]); ++p)
          ent.push_back(Entry{i, p + 1, infos[i].d.out, pass_row_bytes(infos[i], p)});
      } else {
        ent.push_back(Entry{i, 0, infos[i].d.out, row_bytes(infos[i])});
      }
    }
    for (const Entry& e : ent) total += e.rb * e.out;
    const uint32_t ne = (uint32_t)ent.size();
    // Small ranges (a few rows each): a range that would take a few rows of
    // the next entry starts that entry instead, since a workgroup pays a
    // segment's fixed latency per segment; large ranges stay exactly
    // balanced.
    const uint64_t share = total / G, snap = share <= kSnapShareBytes ? share / 2 : 0;
    // boundary b: (entry, row) where the b-th range starts; entry == ne past the end
    auto boundary = [&](uint32_t b, uint32_t* e_out, uint32_t* row) {
      const uint64_t pos = (uint64_t)((unsigned __int128)total * b / G);
      uint64_t acc = 0;
      for (uint32_t e = 0; e < ne; ++e) {
        const uint64_t mb = ent[e].rb * ent[e].out;
        if (pos < acc + mb) {
          if (b > 0 && pos - acc < snap) {   // close to the entry's start
            *e_out = e;
            *row = 0;
            return;
          }
          if (b > 0 && acc + mb - pos < snap) {   // close to the entry's end
            *e_out = e + 1;
            *row = 0;
            return;
          }
          uint64_t r = (pos - acc + ent[e].rb / 2) / ent[e].rb;
          if (ent[e].pass1) r = (r + 8) / 16 * 16;
          *e_out = e;
          *row = (uint32_t)r;
          if (r >= ent[e].out) {   // rounds to the next entry
            *e_out = e + 1;
            *row = 0;
          }
          return;
        }
        acc += mb;
      }
      *e_out = ne;
      *row = 0;
    };
    uint32_t nseg = 0, e0 = 0, r0 = 0;
    boundary(0, &e0, &r0);
    const uint32_t sr = seg_rows(c);
    for (uint32_t b = 0; b < G; ++b) {
      blockseg[b] = nseg;
      uint32_t e1 = 0, r1 = 0;
      boundary(b + 1, &e1, &r1);
      for (uint32_t e = e0; e < ne && e <= e1; ++e) {
        const uint32_t rs = e == e0 ? r0 : 0;
        const uint32_t re = e == e1 ? r1 : ent[e].out;
        for (uint32_t r = rs; r < re; r += sr)
          segs[nseg++] = Seg{ent[e].mat, r, re - r > sr ? r + sr : re, ent[e].pass1};
      }
      e0 = e1;
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
  h->x_dtype = (uint32_t)x_dtype_flags;
  h->zjob_terms = P.zterms;
  h->reserved = P.n_classes;
  h->off_descs = P.off_descs;
  h->off_zjobs = P.off_zjobs;
  h->bytes = P.bytes;

  ginfo->n = n;
  ginfo->n_classes = P.n_classes;
  ginfo->n_segs = nseg_total;
  ginfo->n_zjobs = (uint32_t)j;
  ginfo->x_dtype = (uint32_t)x_dtype_flags;
  ginfo->zjob_terms = P.zterms;
  ginfo->rows_per_batch = kRB;
  ginfo->grid = gmax;
  ginfo->plan_bytes = P.bytes;
  ginfo->off_descs = P.off_descs;
  ginfo->off_zjobs = P.off_zjobs;
  ginfo->sync_dev = plan_syncs(n, infos, P) ? ws_dev : nullptr;
  uint64_t alg = 0;
  for (uint32_t i = 0; i < n; ++i) alg += infos[i].algorithmic_bytes;
  ginfo->algorithmic_bytes = alg;
  return WAL_OK;
}

int wal_gemv_grouped_phases(const wal_grouped_info* g, const void* plan_dev, int phases, void* stream) {
  if (!g || !plan_dev) return WAL_ERR_ARG;
  if (phases < 1 || phases > WAL_PHASE_ALL) return WAL_ERR_ARG;
  if (!aligned(plan_dev, 16)) return WAL_ERR_ALIGN;
  if ((g->x_dtype & ~(uint32_t)(WAL_X_BF16 | WAL_X_ROT_H128)) || !g->n) return WAL_ERR_ARG;
  if (g->rows_per_batch != (uint32_t)kRB || !g->n_classes || g->n_classes > WAL_MAX_CLASSES) return WAL_ERR_ARG;
  for (uint32_t k = 0; k < g->n_classes; ++k) {
    if (g->class_id[k] >= kClasses || !g->class_grid[k]) return WAL_ERR_ARG;
    if (!grouped_for((int)g->x_dtype, g->class_id[k])) return WAL_ERR_UNSUPPORTED;
    if (g->class_blockseg[k] >= g->plan_bytes || g->class_segs[k] >= g->plan_bytes) return WAL_ERR_ARG;
  }
  if (g->off_descs >= g->plan_bytes || (g->n_zjobs && g->off_zjobs >= g->plan_bytes)) return WAL_ERR_ARG;
  if (g->n_zjobs && g->zjob_terms != kZTermsFew && g->zjob_terms != kZTermsMany) return WAL_ERR_ARG;
  if (g->n_zjobs && !g->sync_dev) return WAL_ERR_ARG;
  if (g->sync_dev && !aligned(g->sync_dev, 16)) return WAL_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* base = static_cast<const uint8_t*>(plan_dev);
  const MatDev* descs = reinterpret_cast<const MatDev*>(base + g->off_descs);
  const uint32_t* jobs = reinterpret_cast<const uint32_t*>(base + g->off_zjobs);
  // Both phases: the low-rank jobs run in the first workgroups of the first
  // streaming launch (the plan's synchronisation words order them).
  const bool fused = phases == WAL_PHASE_ALL;
  int st;
  if (!fused && (phases & WAL_PHASE_LOWRANK) && g->n_zjobs) {
    const bool bf16 = (g->x_dtype & WAL_X_BF16) != 0, rot = (g->x_dtype & WAL_X_ROT_H128) != 0;
    auto zk = bf16 ? (rot ? k_z_grouped<WAL_X_BF16, true> : k_z_grouped<WAL_X_BF16, false>)
                   : (rot ? k_z_grouped<WAL_X_F32, true> : k_z_grouped<WAL_X_F32, false>);
    hipLaunchKernelGGL(zk, dim3(g->n_zjobs), dim3(kThreads), 0, s, descs, jobs, g->zjob_terms);
    if ((st = launch_status())) return st;
  }
  uint32_t* sync = static_cast<uint32_t*>(g->sync_dev);
  for (uint32_t k = 0; (phases & WAL_PHASE_STREAM) && k < g->n_classes; ++k) {
    const uint32_t* blockseg = reinterpret_cast<const uint32_t*>(base + g->class_blockseg[k]);
    const Seg* segs = reinterpret_cast<const Seg*>(base + g->class_segs[k]);
    // the synchronisation words also serve split matrices' arrival counts,
    // so every streaming launch of a plan that has them takes them
    const uint32_t nz = fused && sync && k == 0 ? g->n_zjobs : 0u;
    const uint32_t grid = g->class_grid[k] + nz;
    Fuse f{};
    if (sync) f = Fuse{sync, k, nz, nz ? 1u : 0u, grid, k + 1 == g->n_classes ? 1u : 0u, g->zjob_terms};
    hipLaunchKernelGGL(grouped_for((int)g->x_dtype, g->class_id[k]), dim3(grid), dim3(kThreads), 0, s, descs,
                       blockseg, segs, jobs, f);
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
