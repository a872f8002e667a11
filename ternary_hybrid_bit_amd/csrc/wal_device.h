// Device helpers shared by the HIP kernels of libwal (gfx950, wave64):
// cross-lane reductions, buffer resources, scale decoding.
#pragma once

#include <hip/hip_runtime.h>

#include "wal_internal.h"

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x3_t __attribute__((ext_vector_type(3)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

namespace {

using namespace wal;

// ---------------------------------------------------------------------------
// Cross-lane helpers.

template <int CTRL, int ROWMASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

__device__ __forceinline__ void swap32_add(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16_add(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One butterfly level on lane bit `BIT` (3, 2, 1 or 0) for R values: pairs
// v[j] and v[j + H] (H = R >> (6 - BIT)), lanes with the bit set keep the
// second of the pair.
template <int BIT, int CTRL, int R>
__device__ __forceinline__ void tlevel(float (&v)[R], int lane) {
  constexpr int H = R >> (6 - BIT);
  if constexpr (H >= 1) {
    const bool hi = (lane >> BIT) & 1;
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const float a = hi ? v[j + H] : v[j];
      const float b = hi ? v[j] : v[j + H];
      v[j] = a + dpp<CTRL>(b);
    }
  } else {
    v[0] += dpp<CTRL>(v[0]);
  }
}

// Transposed reduction of R per-lane values (R a power of two <= 64): returns,
// in lane l, the wavefront total of value (l >> (6 - log2 R)).
template <int R>
__device__ __forceinline__ float treduce(float (&v)[R], int lane) {
  if constexpr (R >= 2) {
#pragma unroll
    for (int j = 0; j < R / 2; ++j) swap32_add(v[j], v[j + R / 2]);
  } else {
    float w = v[0];
    swap32_add(v[0], w);
  }
  if constexpr (R >= 4) {
#pragma unroll
    for (int j = 0; j < R / 4; ++j) swap16_add(v[j], v[j + R / 4]);
  } else {
    float w = v[0];
    swap16_add(v[0], w);
  }
  tlevel<3, 0x128>(v, lane);   // row_ror:8
  tlevel<2, 0x141>(v, lane);   // row_half_mirror
  tlevel<1, 0x4E>(v, lane);    // quad_perm [2,3,0,1]
  tlevel<0, 0xB1>(v, lane);    // quad_perm [1,0,3,2]
  return v[0];
}

// Sum over aligned groups of L lanes (L = 8, 16, 32 or 64); every lane of a
// group receives the group total.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  if constexpr (L >= 16) v += dpp<0x140>(v);   // row_mirror
  if constexpr (L >= 32) { float w = v; swap16_add(v, w); }
  if constexpr (L >= 64) { float w = v; swap32_add(v, w); }
  return v;
}

// Hand-off of LDS data between the lanes of one wavefront: every lane's LDS
// accesses before the call are ordered before every lane's accesses after
// it.  The release and acquire fences keep the compiler from dropping or
// moving the accesses (a lane reads what other lanes wrote, which its own
// view of memory does not show); the wave barrier is the point every lane
// reaches together.  One wavefront's LDS operations execute in issue order,
// so this emits no instructions.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------
// Buffer loads: a resource over one plane, a per-lane offset and a per-row
// scalar offset.

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// A resource over the activations of one product: loads past the row's end
// (lanes beyond the last pass's width) read zeros without touching memory.
template <int XT>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t x_rsrc(const void* x, uint32_t n) {
  return rsrc(x, n * (XT == WAL_X_F32 ? 4u : 2u));
}

// Activation element as fp32.
template <int XT>
__device__ __forceinline__ float xval(const void* x, uint32_t i) {
  if constexpr (XT == WAL_X_F32) return reinterpret_cast<const float*>(x)[i];
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[i] << 16);
}

// 64-bit left shift by a constant.  Written as an instruction so that the
// compiler does not split it back into two 32-bit shifts (it would, seeing
// that the bits crossing the halves are masked off afterwards).
template <int S>
__device__ __forceinline__ uint64_t shl64(uint64_t v) {
  if constexpr (S == 0) {
    return v;
  } else {
    uint64_t r;
    asm("v_lshlrev_b64 %0, %1, %2" : "=v"(r) : "n"(S), "v"(v));
    return r;
  }
}

// Plane of low-rank path p, from path 0's plane of the same kind.
__device__ __forceinline__ const uint8_t* path_plane(const uint8_t* p0, const MatDev& d, uint32_t p) {
  return p0 + (size_t)p * d.pstride;
}

// ---------------------------------------------------------------------------
// Scales: fp16 (2 bytes) or fp24 (the upper 3 bytes of an fp32 pattern).

// Cache policy of the packed-weight loads: non-temporal.  Every packed byte
// is read once per product, and marking the stream non-temporal lifts a
// plain streaming read on MI355X from about 6.2 to 7.0 TB/s.
constexpr int kStream = 2;

template <int SF>
__device__ __forceinline__ uint32_t load_scale(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (SF == WAL_SCALE_FP16) return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kStream);
  const uint32_t b0 = __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, kStream);
  const uint32_t b1 = __builtin_amdgcn_raw_buffer_load_b8(r, voff + 1, soff, kStream);
  const uint32_t b2 = __builtin_amdgcn_raw_buffer_load_b8(r, voff + 2, soff, kStream);
  return b0 | (b1 << 8) | (b2 << 16);
}

// scale * v + acc in fp32.
template <int SF>
__device__ __forceinline__ float scale_fma(uint32_t raw, float v, float acc) {
  if constexpr (SF == WAL_SCALE_FP16)
    return __builtin_fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)raw), v, acc);
  return __builtin_fmaf(__uint_as_float(raw << 8), v, acc);
}

__device__ __forceinline__ float f16_at(const uint8_t* p, uint32_t i) {
  return (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(p)[i]);
}

// ---------------------------------------------------------------------------
// Low-rank reductions of one matrix by a whole workgroup:
// z[t] = s_p[r] * sum_j (-1)^{V_p[r] bit j} x_j over the columns j in
// [c0, c1) (multiples of 16) for the C terms t0 .. t0 + C - 1 (those below
// d.terms), written to out[t] by threads t - t0.  Every thread of the
// workgroup (up to 1024) calls it (it holds a barrier).
template <int XT, int C>
__device__ __forceinline__ void z_chunk(const MatDev& d, const void* x, uint32_t t0, float* out, uint32_t c0,
                                        uint32_t c1) {
  __shared__ float red[16][C];
  const uint32_t tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63;
  const uint32_t T = d.terms, vrow = d.in / 8;
  // the per-rank scale of the thread's term, loaded before the sweep so its
  // latency is not paid after the barrier
  // (every thread loads a valid scale, without a branch, so that nothing
  // waits for it before the end)
  uint32_t scale_bits;
  {
    const uint32_t t = min(t0 + (tid < (uint32_t)C ? tid : 0u), T - 1);
    const uint32_t p = t / d.rank, r = t % d.rank;
    scale_bits = reinterpret_cast<const uint16_t*>(path_plane(d.s, d, p))[r];
  }
  float acc[C];
#pragma unroll
  for (int q = 0; q < C; ++q) acc[q] = 0.f;
  // columns c .. c + 15 of the C terms
  auto step = [&](uint32_t c) {
    uint32_t xb[16];   // fp32 bit patterns of x[c .. c + 15]
    if constexpr (XT == WAL_X_BF16) {
      const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + c);
      const uint4 a = src[0], b = src[1];
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        xb[2 * k] = w[k] << 16;
        xb[2 * k + 1] = w[k] & 0xFFFF0000u;
      }
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + c);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 v = src[k];
        xb[4 * k] = v.x; xb[4 * k + 1] = v.y; xb[4 * k + 2] = v.z; xb[4 * k + 3] = v.w;
      }
    }
    // the sign words of all C terms first (terms past the last one read the
    // last term's word, unused), so their latencies overlap
    uint32_t bits[C];
#pragma unroll
    for (int q = 0; q < C; ++q) {
      const uint32_t t = min(t0 + q, T - 1);
      const uint32_t p = t / d.rank, r = t % d.rank;
      bits[q] = reinterpret_cast<const uint16_t*>(path_plane(d.V, d, p) + (size_t)r * vrow)[c / 16];
    }
#pragma unroll
    for (int q = 0; q < C; ++q) {
      if (t0 + q < T) {
        // a set bit flips the sign of x_j
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[q] += __uint_as_float(xb[j] ^ ((bits[q] << (31 - j)) & 0x80000000u));
      }
    }
  };
  // The first step is written out before the loop: its loads then follow
  // the scale's at once (a loop head would wait for every load in flight).
  uint32_t c = c0 + tid * 16;
  if (c < c1) step(c);
  for (c += nthr * 16; c < c1; c += nthr * 16) step(c);
  const float tot = treduce<C>(acc, lane);
  constexpr int SH = 6 - ilog2(C);
  if ((lane & ((1 << SH) - 1)) == 0) red[tid >> 6][lane >> SH] = tot;
  __syncthreads();
  if (tid < (uint32_t)C) {
    const uint32_t t = t0 + tid;
    if (t < T) {
      float sum = 0.f;
      for (uint32_t w = 0; w < (nthr >> 6); ++w) sum += red[w][tid];
      out[t] = (float)__builtin_bit_cast(_Float16, (uint16_t)scale_bits) * sum;
    }
  }
}

// The low-rank reductions a streaming workgroup needs, z[t] for t < d.terms,
// are the sums of d.zc partials (one per column chunk).  A thread first issues
// the loads of up to ZP partials of its term (prefetch) and adds them later
// (total), so the loads overlap other memory latency.
template <int ZP>
struct ZPart {
  float v[ZP];
};

// Only when d.terms > 0.  Threads past the last term load the last term's
// partials (unused) rather than branch.
template <int ZP>
__device__ __forceinline__ void z_prefetch(const MatDev& d, uint32_t t, ZPart<ZP>& zp) {
  const uint32_t tt = t < d.terms ? t : d.terms - 1;
  const __amdgpu_buffer_rsrc_t rz = rsrc(d.z, 4 * d.zc * d.terms);
#pragma unroll
  for (int cc = 0; cc < ZP; ++cc)
    zp.v[cc] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rz, 4 * (cc * d.terms + tt), 0, 0));
}

// Partials in chunk order (a fixed order: results do not depend on timing).
// Chunks past d.zc read as zero (out of the resource's range).
template <int ZP>
__device__ __forceinline__ float z_total(const MatDev& d, uint32_t t, const ZPart<ZP>& zp) {
  float z = zp.v[0];
#pragma unroll
  for (int cc = 1; cc < ZP; ++cc) z += zp.v[cc];
  for (uint32_t cc = ZP; cc < d.zc; ++cc) z += d.z[cc * d.terms + t];
  return z;
}


}  // namespace
