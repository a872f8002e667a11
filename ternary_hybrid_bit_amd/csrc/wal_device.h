// Device helpers shared by the HIP kernels of libwal (gfx950, wave64):
// cross-lane reductions, buffer resources, scale decoding.
#pragma once

#include <hip/hip_runtime.h>

#include "wal_internal.h"

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x3_t __attribute__((ext_vector_type(3)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

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
// Normalised Hadamard-128 rotation of the activations (WAL2-Ternary-27B card,
// "Архитектура": a blob stored as W' = W R, R = blockdiag(H / sqrt(128)) with
// H Sylvester's Hadamard matrix, takes x~ = R x).
//
// out[128 g + i] = fp32(1/sqrt(128)) * (sum_j H[i][j] x[128 g + j]), the sum
// as butterflies (a, b) -> (a + b, a - b) in fp32 over column bits 0..3
// inside a thread (16 consecutive values), then bits 4, 5, 6 between the
// eight threads of the group, in that order; bf16 activations are rounded to
// nearest even afterwards.  wal_rotate_h128 runs the same steps, so a product
// that rotates its own x gives the bits of the rotate-then-multiply pair.
//
// Inside a product the workgroup (256 threads) rotates 32 groups per round.
// The eight threads of a group are lanes {0, 1, 2, 3, 8, 9, 10, 11} (or the
// same + 4) of one 16-lane row, so that column bits 4, 5 and 6 sit at lane
// bits 0, 1 and 3 and every partner is one DPP move away: xor 1 and xor 2
// are quad permutations, xor 8 the row rotation by 8.
constexpr float kInvSqrt128 = 0.08838834764831845f;   // 1 / sqrt(128), rounded to fp32

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;   // NaN stays NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// The thread's piece of round r: group g of the round's columns, columns
// 16 sub .. 16 sub + 15 of it.
struct RotSlot {
  uint32_t g, sub;
};
__device__ __forceinline__ RotSlot rot_slot(uint32_t round) {
  static_assert(kThreads == 256, "32 groups per round of a 256-thread workgroup");
  const uint32_t l = threadIdx.x & 63, w = threadIdx.x >> 6;
  return RotSlot{32 * round + 2 * (4 * w + (l >> 4)) + ((l >> 2) & 1), (l & 3) | (((l >> 3) & 1) << 2)};
}

// The 16 activations of a piece starting at column col, as fp32 (columns
// past the resource's end read as zero).
template <int XT>
__device__ __forceinline__ void rot_load(__amdgpu_buffer_rsrc_t rx, uint32_t col, float (&v)[16]) {
  if constexpr (XT == WAL_X_BF16) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(rx, 2 * col + 16 * h, 0, 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * h + 2 * k] = __uint_as_float(w[k] << 16);
        v[8 * h + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(rx, 4 * col + 16 * h, 0, 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) v[4 * h + k] = __uint_as_float(w[k]);
    }
  }
}

// One cross-lane level: the thread whose column bit is set keeps p - v, the
// other v + p (p the partner's value), both as one DPP add of a sign-flipped
// own value.
template <int CTRL>
__device__ __forceinline__ void rot_level(float (&v)[16], bool second) {
  const uint32_t flip = second ? 0x80000000u : 0u;
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = dpp<CTRL>(v[j]) + __uint_as_float(__float_as_uint(v[j]) ^ flip);
}

// The rotated values of the thread's piece: the butterflies, the scale, and
// for bf16 activations the rounding (values stay fp32 holding bf16 values).
template <int XT>
__device__ __forceinline__ void rot_apply(float (&v)[16], uint32_t sub) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (!(j & h)) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
  rot_level<0xB1>(v, sub & 1);    // quad_perm [1,0,3,2]: column bit 4
  rot_level<0x4E>(v, sub & 2);    // quad_perm [2,3,0,1]: column bit 5
  rot_level<0x128>(v, sub & 4);   // row_ror:8: column bit 6
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    v[j] *= kInvSqrt128;
    if constexpr (XT == WAL_X_BF16) v[j] = __uint_as_float(bf16_rne(v[j]) << 16);
  }
}

// The piece as activations of x's type at element e of xs (LDS).
template <int XT>
__device__ __forceinline__ void rot_store_x(void* xs, uint32_t e, const float (&v)[16]) {
  if constexpr (XT == WAL_X_BF16) {
    uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(xs) + e);
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = (__float_as_uint(v[2 * k]) >> 16) | (__float_as_uint(v[2 * k + 1]) & 0xFFFF0000u);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(xs) + e);
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
}

// The piece's entries of a signed site table tbl[group][site byte]: +-2x for
// bf16 activations, +-x for fp32 (the streaming kernels' scaling).
template <int XT>
__device__ __forceinline__ void rot_store_tbl(float* tbl, const RotSlot& s, const float (&v)[16]) {
  constexpr float m = XT == WAL_X_BF16 ? 2.0f : 1.0f;
  float4* pos = reinterpret_cast<float4*>(tbl + s.g * 256 + 16 * s.sub);
  float4* neg = reinterpret_cast<float4*>(tbl + s.g * 256 + 128 + 16 * s.sub);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = m * v[4 * k], b = m * v[4 * k + 1], c = m * v[4 * k + 2], d = m * v[4 * k + 3];
    pos[k] = make_float4(a, b, c, d);
    neg[k] = make_float4(-a, -b, -c, -d);
  }
}

// ---------------------------------------------------------------------------
// The same rotation of bf16 activations on the matrix cores: rotating groups
// is a dense product X H (rows of X the groups, H the 128 x 128 +-1 matrix),
// exact in its bf16 operands and summed in fp32, which costs each wavefront
// a few MFMAs instead of hundreds of vector instructions per piece.
//
// A 16-group x 16-column tile is four v_mfma_f32_16x16x32_bf16 along the
// input column k = 32 s + 8 kb + e (step s): x is the A operand (lane (i, kb)
// holds x[group i][32 s + 8 kb .. + 7], 16 contiguous bytes), H the B operand
// (lane (n, kb) holds H[32 s + 8 kb + e][16 jt + n] for e = 0..7), and lane
// (n, q) ends with groups 4 q .. 4 q + 3 of output column 16 jt + n.  The
// sign of H[k][j] is the parity of popcount(e & n) + kb0 n3 + kb1 jt0 +
// s0 jt1 + s1 jt2; wavefront w takes the column tiles jt = w + 4 u (u = 0, 1),
// so jt0 and jt1 are its own and jt2 = u is known at compile time: four B
// registers per lane serve every tile.  The scale and the bf16 rounding
// (v_cvt_pk_bf16_f32, to nearest even) follow, as in wal_rotate_h128, which
// runs this same code for bf16 input, so the two agree bit for bit.
struct RotB {
  uint4 even, even_neg, odd, odd_neg;   // B operands of even / odd steps s

  __device__ __forceinline__ void init() {
    const uint32_t l = threadIdx.x & 63, n = l & 15, kb = l >> 4, w = wave_id();
    uint32_t p[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t v = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t e = 2 * q + h;
        const uint32_t neg = (__builtin_popcount(e & n) + (kb & 1) * (n >> 3) + ((kb >> 1) & w & 1)) & 1;
        v |= (0x3F80u | (neg << 15)) << (16 * h);
      }
      p[q] = v;
    }
    const uint32_t odd_flip = (w & 2) ? 0x80008000u : 0u;   // s0 jt1, jt1 = bit 1 of w
    even = make_uint4(p[0], p[1], p[2], p[3]);
    even_neg = make_uint4(p[0] ^ 0x80008000u, p[1] ^ 0x80008000u, p[2] ^ 0x80008000u, p[3] ^ 0x80008000u);
    odd = make_uint4(p[0] ^ odd_flip, p[1] ^ odd_flip, p[2] ^ odd_flip, p[3] ^ odd_flip);
    odd_neg = make_uint4(odd.x ^ 0x80008000u, odd.y ^ 0x80008000u, odd.z ^ 0x80008000u, odd.w ^ 0x80008000u);
  }
  // step S of column tile w + 4 U: the s1 jt2 sign is S >> 1 & U
  template <int S, int U>
  __device__ __forceinline__ const uint4& op() const {
    constexpr bool neg = ((S >> 1) & U) != 0;
    if constexpr (S & 1) return neg ? odd_neg : odd;
    return neg ? even_neg : even;
  }
};

__device__ __forceinline__ f32x4_t rot_mfma(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// NGT tiles of 16 groups (groups 16 gt + i) of one row of bf16 activations,
// rotated: load the x operands, compute (rounded to bf16), then store.
template <int NGT, bool F32OUT = false>
struct RotTiles {
  uint4 a[NGT][4];       // x operands [group tile][step]
  uint32_t r[NGT][2][2];  // results as bf16 pairs: [group tile][u][pair of groups 4 q + (0, 1) / (2, 3)]
  f32x4_t f[F32OUT ? NGT : 1][2];   // with F32OUT: the scaled fp32 results [group tile][u]

  // Group g's columns start at element col0 + 128 g of the resource; groups
  // g >= ng load zeros.
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rx, uint32_t col0, uint32_t ng) {
    const uint32_t l = threadIdx.x & 63, i = l & 15, kb = l >> 4;
#pragma unroll
    for (int gt = 0; gt < NGT; ++gt) {
      const uint32_t g = 16 * gt + i;
      // an offset past 2 GB reads zeros without touching memory
      const uint32_t off = g < ng ? 2 * (col0 + 128 * g + 8 * kb) : 0x80000000u;
#pragma unroll
      for (int s = 0; s < 4; ++s) a[gt][s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off + 64 * s, 0, 0));
    }
  }
  template <int GT, int U>
  __device__ __forceinline__ f32x4_t tile(const RotB& hb) const {
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
    c = rot_mfma(a[GT][0], hb.op<0, U>(), c);
    c = rot_mfma(a[GT][1], hb.op<1, U>(), c);
    c = rot_mfma(a[GT][2], hb.op<2, U>(), c);
    c = rot_mfma(a[GT][3], hb.op<3, U>(), c);
    return c;
  }
  template <int GT>
  __device__ __forceinline__ void compute_from(const RotB& hb) {
    if constexpr (GT < NGT) {
      const f32x4_t c0 = tile<GT, 0>(hb), c1 = tile<GT, 1>(hb);
      if constexpr (F32OUT) {
        f[GT][0] = c0 * kInvSqrt128;
        f[GT][1] = c1 * kInvSqrt128;
        compute_from<GT + 1>(hb);
        return;
      }
      r[GT][0][0] = pack_bf16(c0[0] * kInvSqrt128, c0[1] * kInvSqrt128);
      r[GT][0][1] = pack_bf16(c0[2] * kInvSqrt128, c0[3] * kInvSqrt128);
      r[GT][1][0] = pack_bf16(c1[0] * kInvSqrt128, c1[1] * kInvSqrt128);
      r[GT][1][1] = pack_bf16(c1[2] * kInvSqrt128, c1[3] * kInvSqrt128);
      compute_from<GT + 1>(hb);
    }
  }
  __device__ __forceinline__ void compute() {
    RotB hb;
    hb.init();
    compute_from<0>(hb);
  }
  static __device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  // The rotated value of tile (gt, u), group 4 q + jj, as bf16 bits.
  __device__ __forceinline__ uint32_t bits(int gt, int u, int jj) const {
    return jj & 1 ? r[gt][u][jj >> 1] >> 16 : r[gt][u][jj >> 1] & 0xFFFFu;
  }
  // Output column of tile u for this lane, and group of (gt, jj).
  static __device__ __forceinline__ uint32_t column(int u) { return 16 * (wave_id() + 4 * u) + (threadIdx.x & 15); }
  static __device__ __forceinline__ uint32_t group(int gt, int jj) {
    return 16 * gt + 4 * ((threadIdx.x & 63) >> 4) + jj;
  }

  // Compact activations xs[128 g + j] (bf16, LDS) of groups g < ng.  The
  // lane's first element is 128 (4 q) + 16 w + n; every value sits a
  // constant offset from it (folded into the LDS store).
  __device__ __forceinline__ void store_x(uint16_t* xs, uint32_t ng) const {
    const uint32_t l = threadIdx.x & 63, q = l >> 4;
    uint16_t* base = xs + 512 * q + 16 * wave_id() + (l & 15);
#pragma unroll
    for (int gt = 0; gt < NGT; ++gt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if (16 * gt + 16 <= (int)ng || 16 * gt + 4 * q + jj < ng) {
#pragma unroll
          for (int u = 0; u < 2; ++u) base[128 * (16 * gt + jj) + 64 * u] = (uint16_t)bits(gt, u, jj);
        }
      }
  }
  // Signed site table entries tbl[g][j] = 2 x~, tbl[g][128 + j] = -2 x~ of
  // groups g < ng.
  __device__ __forceinline__ void store_tbl(float* tbl, uint32_t ng) const {
    const uint32_t l = threadIdx.x & 63, q = l >> 4;
    float* base = tbl + 1024 * q + 16 * wave_id() + (l & 15);
#pragma unroll
    for (int gt = 0; gt < NGT; ++gt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if (16 * gt + 16 <= (int)ng || 16 * gt + 4 * q + jj < ng) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float v = __uint_as_float(bits(gt, u, jj) << 16);
            base[256 * (16 * gt + jj) + 64 * u] = 2.0f * v;
            base[256 * (16 * gt + jj) + 64 * u + 128] = -2.0f * v;
          }
        }
      }
  }
};

// The rotation of one pass of NG groups inside a streaming workgroup, in
// three steps around its set-up barriers: load (before the first batch's
// loads), compute (registers only), store the compact activations and the
// signed site table (after the barrier).  bf16 activations go through the
// matrix cores; fp32 activations (NG = 32) through the butterflies, one
// 16-column piece per thread.
template <int XT, int NG>
struct RotPass;

template <int NG>
struct RotPass<WAL_X_BF16, NG> {
  RotTiles<(NG + 15) / 16> t;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rx, uint32_t col0) { t.load(rx, col0, NG); }
  __device__ __forceinline__ void compute() { t.compute(); }
  __device__ __forceinline__ void store_x(void* xs) const { t.store_x(static_cast<uint16_t*>(xs), NG); }
  // table slots: groups < slots (slots past NG receive zeros)
  __device__ __forceinline__ void store_tbl(float* tbl, uint32_t slots) const { t.store_tbl(tbl, slots); }
};

template <int NG>
struct RotPass<WAL_X_F32, NG> {
  static_assert(NG == 32, "fp32 activations: one 4096-column pass of the 2-bit kernels");
  RotSlot s;
  float v[16];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rx, uint32_t col0) {
    s = rot_slot(0);
    rot_load<WAL_X_F32>(rx, col0 + 128 * s.g + 16 * s.sub, v);
  }
  __device__ __forceinline__ void compute() { rot_apply<WAL_X_F32>(v, s.sub); }
  __device__ __forceinline__ void store_x(void* xs) const { rot_store_x<WAL_X_F32>(xs, 128 * s.g + 16 * s.sub, v); }
  __device__ __forceinline__ void store_tbl(float* tbl, uint32_t) const { rot_store_tbl<WAL_X_F32>(tbl, s, v); }
};

// Columns [c0, c0 + 128 ng) of x (n columns; ng <= 64) rotated into xs (LDS,
// x's type, column c0 at element 0) by the whole workgroup, then a barrier.
// Every thread calls it.
template <int XT>
__device__ __forceinline__ void rot_to_lds(const void* x, uint32_t n, uint32_t c0, uint32_t ng, void* xs) {
  const __amdgpu_buffer_rsrc_t rx = rsrc(x, n * (XT == WAL_X_F32 ? 4u : 2u));
  if constexpr (XT == WAL_X_BF16) {
    for (uint32_t g0 = 0; g0 < ng; g0 += 32) {
      RotTiles<2> rt;
      rt.load(rx, c0 + 128 * g0, ng - g0);
      rt.compute();
      rt.store_x(static_cast<uint16_t*>(xs) + 128 * g0, ng - g0);
    }
  } else {
    for (uint32_t round = 0; 32 * round < ng; ++round) {
      const RotSlot s = rot_slot(round);
      float v[16];
      rot_load<XT>(rx, c0 + 128 * s.g + 16 * s.sub, v);
      rot_apply<XT>(v, s.sub);
      if (s.g < ng) rot_store_x<XT>(xs, 128 * s.g + 16 * s.sub, v);
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Data that workgroups of one launch hand to each other (low-rank partials,
// per-pass partial sums) moves through device-scope (agent) atomic stores
// and loads: on this part they go to the device's coherence point, past the
// CU and XCD caches, so a consumer that has seen the producer's count (or
// tag) sees the data without cache maintenance.  The producer's wave waits
// for its own stores to complete (wait_stores) before a count is raised;
// agent-scope release and acquire fences would instead write back or
// invalidate the whole L2 of an XCD, which costs microseconds per workgroup
// here.
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(0): the wave's vector memory operations, stores included,
// have completed.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Low-rank partials that a fused launch hands over carry a tag in the same
// 64-bit word (one device-scope store and load each): a consumer that reads
// a partial with the call's tag has its value, so one read both checks and
// fetches it.
__device__ __forceinline__ void store_tagged(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_tagged(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float tagged_value(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ uint32_t tagged_tag(uint64_t w) { return (uint32_t)(w >> 32); }

// Where z_chunk writes: LDS floats, device floats (device-scope stores), or
// tagged device words (with the tag read from *epoch: 2 epoch + 1; tag 0
// without an epoch).
enum ZOut { kZOutLds, kZOutDev, kZOutTagged };

// ---------------------------------------------------------------------------
// Low-rank reductions of one matrix by a whole workgroup:
// z[t] = s_p[r] * sum_j (-1)^{V_p[r] bit j} x_j over the columns j in
// [c0, c1) (multiples of 16) for the C terms t0 .. t0 + C - 1 (those below
// d.terms), written to out[t] by threads t - t0 as OUT says (out: float* for
// floats, uint64_t* for tagged words).  Column c is element c - xoff of x
// (a rotated chunk in LDS starts at its first column).  Every thread of the
// workgroup (up to 1024) calls it (it holds a barrier).
template <int XT, int C, ZOut OUT>
__device__ __forceinline__ void z_chunk(const MatDev& d, const void* x, uint32_t t0, void* out, uint32_t c0,
                                        uint32_t c1, const uint32_t* epoch = nullptr, uint32_t xoff = 0) {
  __shared__ float red[16][C];
  const uint32_t tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63;
  const uint32_t T = d.terms, vrow = d.in / 8;
  // the writers' tag, read before the sweep (its latency overlaps it)
  uint32_t tag = 0;
  if constexpr (OUT == kZOutTagged)
    if (epoch && tid < (uint32_t)C) tag = (__hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) << 1) | 1u;
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
      const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + (c - xoff));
      const uint4 a = src[0], b = src[1];
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        xb[2 * k] = w[k] << 16;
        xb[2 * k + 1] = w[k] & 0xFFFF0000u;
      }
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + (c - xoff));
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
      const float v = (float)__builtin_bit_cast(_Float16, (uint16_t)scale_bits) * sum;
      if constexpr (OUT == kZOutLds) static_cast<float*>(out)[t] = v;
      else if constexpr (OUT == kZOutDev) store_dev(static_cast<float*>(out) + t, v);
      else store_tagged(static_cast<uint64_t*>(out) + t, v, tag);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused launches: the low-rank pre-pass in the first workgroups of the
// streaming launch (see Fuse in wal_internal.h).  Producers write their jobs'
// partials as tagged words (store_tagged) with the call's tag; consumers, in
// their epilogue after their streaming, read the partials they need and
// retry (bounded) until every one carries the tag.  Each word that the whole
// launch touches is read and written through the workgroup's copy
// (blockIdx.x % kSyncReplicas).

constexpr uint32_t kSpinLimit = 1u << 16;   // reads of a bounded wait (tens of ms)

// Low-rank jobs as the producers of a launch run them: f.zterms terms of one
// column chunk of kCols columns each (single products: kZTermsFew terms;
// grouped plans: kZTermsFew or kZTermsMany, as planned).  The fallback of a
// consumer whose wait gave up runs the same jobs, so its terms are
// bit-identical.
template <uint32_t COLS, bool TWO_SIZES>
struct ZJobs {
  static constexpr uint32_t kCols = COLS;
  static constexpr bool kTwoSizes = TWO_SIZES;
};
using ZJobsSingle = ZJobs<kZSingleCols, false>;
using ZJobsGrouped = ZJobs<kZChunkCols, true>;

template <class ZJ>
__device__ __forceinline__ uint32_t zjob_terms(const Fuse& f) {
  return ZJ::kTwoSizes && f.zterms == kZTermsMany ? kZTermsMany : kZTermsFew;
}

// The terms t0 .. t0 + C - 1 of a job over columns [c0, c1): from x, or in a
// rotated product (ROT) from the chunk rotated into xs (LDS, at least
// c1 - c0 activations of x's type) first.  Every thread calls it.
template <int XT, int C, ZOut OUT, bool ROT>
__device__ __forceinline__ void z_chunk_rot(const MatDev& d, uint32_t t0, void* out, uint32_t c0, uint32_t c1,
                                            const uint32_t* epoch, void* xs) {
  if constexpr (ROT) {
    rot_to_lds<XT>(d.x, d.in, c0, (c1 - c0) / 128, xs);
    z_chunk<XT, C, OUT>(d, xs, t0, out, c0, c1, epoch, c0);
  } else {
    z_chunk<XT, C, OUT>(d, d.x, t0, out, c0, c1, epoch);
  }
}

// One job: terms t0 .. t0 + terms - 1 over columns [c0, c1) into out (xs:
// LDS for a rotated chunk).
template <int XT, class ZJ, ZOut OUT, bool ROT>
__device__ __forceinline__ void z_job(const MatDev& d, uint32_t terms, uint32_t t0, void* out, uint32_t c0,
                                      uint32_t c1, const uint32_t* epoch, void* xs) {
  if constexpr (ZJ::kTwoSizes) {
    if (terms == kZTermsMany) {
      z_chunk_rot<XT, (int)kZTermsMany, OUT, ROT>(d, t0, out, c0, c1, epoch, xs);
      return;
    }
  }
  z_chunk_rot<XT, (int)kZTermsFew, OUT, ROT>(d, t0, out, c0, c1, epoch, xs);
}

__device__ __forceinline__ uint32_t* sync_copy(const Fuse& f, uint32_t word) {
  return f.sync + word + kSyncLine * (blockIdx.x % kSyncReplicas);
}

// The epoch copy a producer's tag comes from (null: untagged, tag 0).
__device__ __forceinline__ const uint32_t* epoch_of(const Fuse& f) {
  return f.sync ? sync_copy(f, kSyncEpoch) : nullptr;
}

// The last workgroup of the launch to finish returns its slot's words to
// zero and, after the call's last launch, clears the gave-up word and moves
// every epoch copy to one past its own (which also mends copies that
// disagree).  Copy r counts the workgroups b % kSyncReplicas == r; the one
// that completes a copy counts it in line 0, and the one that completes the
// last copy resets.  No data changes hands here: the counts order nothing
// but the reset.  Every thread calls it; thread `counter` does the counting
// (its wave waits for the counts' round trips).
__device__ __forceinline__ void finish_launch(const Fuse& f, uint32_t counter = 0) {
  if (!f.sync) return;
  __syncthreads();
  if (threadIdx.x == counter) {
    const uint32_t r = blockIdx.x % kSyncReplicas;
    const uint32_t members = (f.grid - r + kSyncReplicas - 1) / kSyncReplicas;
    const uint32_t copies = min(f.grid, kSyncReplicas);
    const uint32_t done = __hip_atomic_fetch_add(sync_copy(f, kSyncFinished + f.slot), 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (done + 1 == members &&
        __hip_atomic_fetch_add(f.sync + kSyncSlotsDone + f.slot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 ==
            copies) {
      for (uint32_t c = 0; c < copies; ++c)
        __hip_atomic_store(f.sync + kSyncFinished + kSyncLine * c + f.slot, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(f.sync + kSyncSlotsDone + f.slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (f.last) {
        const uint32_t next = __hip_atomic_load(sync_copy(f, kSyncEpoch), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
        for (uint32_t c = 0; c < kSyncReplicas; ++c)
          __hip_atomic_store(f.sync + kSyncEpoch + kSyncLine * c, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(f.sync + kSyncGaveUp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The end of a streaming segment: ybuf[i] holds the product of row row0 + i
// over every pass, without the low-rank term.
//
// Low-rank term: U_p's byte b of a row holds the signs of terms 8 b .. 8 b
// + 7 of path p, so the row's term is sum over (p, b) of T_pb[byte], with
// table T_pb[u] = sum_k (bit k of u ? -z : +z)[p, 8 b + k].  The tables (one
// per path and U byte, 256 floats each) are built in `tbl` (the site table,
// free by then) from z, the sum of the d.zc low-rank partials in chunk order;
// each row then adds one entry per U byte, in (p, b) order.  Every sum runs in
// a fixed order.
struct SegEnd {
  float* tbl;    // >= n_paths * ceil(rank / 8) * 256 floats of LDS
  float* z;      // >= terms floats of LDS
  float* ybuf;   // LDS, the segment's rows
};

// One read of the partials of term t: their sum in chunk order, and whether
// each carries `tag` (tag 0: any).  Up to kAhead chunks are loaded before
// any is used, so they cost one round trip.
__device__ __forceinline__ bool read_partials(const MatDev& d, uint32_t t, uint32_t tag, float* sum) {
  constexpr uint32_t kAhead = 4;
  const uint64_t* zt = reinterpret_cast<const uint64_t*>(d.z) + t;
  uint64_t w[kAhead];
#pragma unroll
  for (uint32_t k = 0; k < kAhead; ++k) w[k] = k < d.zc ? load_tagged(zt + (size_t)k * d.terms) : 0;
  float z = 0.f;
  bool ok = true;
#pragma unroll
  for (uint32_t k = 0; k < kAhead; ++k) {
    if (k < d.zc) {
      z += tagged_value(w[k]);
      ok = ok && (tag == 0 || tagged_tag(w[k]) == tag);
    }
  }
  for (uint32_t k = kAhead; k < d.zc; ++k) {
    const uint64_t v = load_tagged(zt + (size_t)k * d.terms);
    z += tagged_value(v);
    ok = ok && (tag == 0 || tagged_tag(v) == tag);
  }
  *sum = z;
  return ok;
}

// The fallback of a consumer whose wait gave up: z computed here, one thread
// per term over every column in order (few registers: it must not weigh on
// the streaming code that shares its kernel; it runs only if a wait expires,
// and its sums, in another order than the producers', agree with theirs to
// rounding).  Every thread calls it.
template <int XT, bool ROT>
__device__ __forceinline__ void lowrank_z_here(const MatDev& d, const SegEnd& e) {
  const uint32_t vrow = d.in / 8;
  if constexpr (ROT) {
    // Rotated activations: 4096 columns at a time rotated into the table's
    // space (free here), one thread per term (at most kThreads terms).
    const uint32_t t = threadIdx.x;
    const uint32_t p = t < d.terms ? t / d.rank : 0, r = t < d.terms ? t % d.rank : 0;
    const uint16_t* bits = reinterpret_cast<const uint16_t*>(path_plane(d.V, d, p) + (size_t)r * vrow);
    float z = 0.f;
    for (uint32_t c0 = 0; c0 < d.in; c0 += kPass2bit) {
      const uint32_t nc = min(kPass2bit, d.in - c0);
      rot_to_lds<XT>(d.x, d.in, c0, nc / 128, e.tbl);
      if (t < d.terms) {
        for (uint32_t c = 0; c < nc; c += 16) {
          const uint32_t v = bits[(c0 + c) / 16];
          for (uint32_t j = 0; j < 16; ++j) {
            float xj;
            if constexpr (XT == WAL_X_BF16)
              xj = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(e.tbl)[c + j] << 16);
            else
              xj = e.tbl[c + j];
            z += ((v >> j) & 1u) ? -xj : xj;
          }
        }
      }
      __syncthreads();   // the chunk's readers are done
    }
    if (t < d.terms)
      e.z[t] = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(path_plane(d.s, d, p))[r]) * z;
    return;
  }
  for (uint32_t t = threadIdx.x; t < d.terms; t += blockDim.x) {
    const uint32_t p = t / d.rank, r = t % d.rank;
    const uint16_t* bits = reinterpret_cast<const uint16_t*>(path_plane(d.V, d, p) + (size_t)r * vrow);
    float z = 0.f;
    for (uint32_t c = 0; c < d.in; c += 16) {
      const uint32_t v = bits[c / 16];
      for (uint32_t j = 0; j < 16; ++j) {
        float xj;
        if constexpr (XT == WAL_X_BF16)
          xj = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(d.x)[c + j] << 16);
        else
          xj = reinterpret_cast<const float*>(d.x)[c + j];
        z += ((v >> j) & 1u) ? -xj : xj;
      }
    }
    e.z[t] = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(path_plane(d.s, d, p))[r]) * z;
  }
}

// z = the sum of the low-rank partials in chunk order, from the workspace:
// with f.zwait, read until every partial carries the call's tag (the tag,
// from the epoch, is read in the same round trip) — bounded.  False when the
// wait gave up (then the caller computes z with lowrank_z_here).  Every
// thread calls it (barriers).
__device__ __forceinline__ bool lowrank_z_read(const MatDev& d, const SegEnd& e, const Fuse& f) {
  const uint32_t t = threadIdx.x;
  __shared__ uint32_t s_miss, s_give;
  const uint32_t* ep = f.zwait ? sync_copy(f, kSyncEpoch) : nullptr;
  for (uint32_t n = 1;; ++n) {
    if (t == 0) s_miss = 0;
    __syncthreads();
    if (t < d.terms) {
      const uint32_t tag = ep ? (__hip_atomic_load(ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) << 1) | 1u : 0u;
      float z;
      if (!read_partials(d, t, tag, &z)) s_miss = 1;
      e.z[t] = z;
    }
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(s_miss)) return true;
    // not all there yet: read again, bounded; on expiry, or once another
    // workgroup of the call gave up, compute the terms here
    if (t == 0) {
      const bool give = n == kSpinLimit || __hip_atomic_load(f.sync + kSyncGaveUp, __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT);
      if (give) {
        __hip_atomic_store(f.sync + kSyncGaveUp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(f.sync + kSyncFallback, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      s_give = give;
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(s_give)) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// The byte tables from z: thread u builds entry u of every table.  Every
// thread calls it (barrier).
__device__ __forceinline__ void lowrank_build(const MatDev& d, const SegEnd& e) {
  const uint32_t ub = (d.rank + 7) / 8;
  for (uint32_t u = threadIdx.x; u < 256; u += blockDim.x) {
    float* out = e.tbl + u;
    const float* z = e.z;
    for (uint32_t p = 0; p < d.n_paths; ++p, z += d.rank)
      for (uint32_t b = 0; b < ub; ++b, out += 256) {
        float sum = 0.f;
        for (uint32_t k = 0; k < 8 && 8 * b + k < d.rank; ++k) sum += ((u >> k) & 1u) ? -z[8 * b + k] : z[8 * b + k];
        *out = sum;
      }
  }
  __syncthreads();
}

// The U bytes of one row, loaded ahead of the tables: per path the eight
// bytes from the dword holding the row's first U byte (a row's ub <= 4 U
// bytes per path then lie inside them).  Reads past the blob return zero.
constexpr uint32_t kUAheadPaths = 2;
struct UAhead {
  uint64_t w[kUAheadPaths];
  uint32_t sh;   // bit offset of the row's first byte in each window
};

// rows of at most 4 U bytes per path and at most kUAheadPaths paths
__device__ __forceinline__ bool u_ahead_fits(const MatDev& d) { return d.rank <= 32 && d.n_paths <= kUAheadPaths; }

__device__ __forceinline__ UAhead load_u_ahead(const MatDev& d, __amdgpu_buffer_rsrc_t ru, uint32_t row) {
  const uint32_t ub = (d.rank + 7) / 8, o = (uint32_t)(d.U - d.codes) + row * ub;
  UAhead u;
  u.sh = 8 * (o & 3u);
#pragma unroll
  for (uint32_t p = 0; p < kUAheadPaths; ++p) {
    const uint32_t a = (o & ~3u) + p * d.pstride;
    const uint32_t lo = p < d.n_paths ? __builtin_amdgcn_raw_buffer_load_b32(ru, a, 0, 0) : 0u;
    const uint32_t hi = p < d.n_paths ? __builtin_amdgcn_raw_buffer_load_b32(ru, a + 4, 0, 0) : 0u;
    u.w[p] = ((uint64_t)hi << 32) | lo;
  }
  return u;
}

// Low-rank term of a row from its U bytes loaded ahead: from the byte
// tables, or (direct) from z with the tables' own arithmetic, entry by entry
// in the same order, so both give the same bits.
template <bool DIRECT>
__device__ __forceinline__ float lowrank_row_ahead(const MatDev& d, const SegEnd& e, const UAhead& u) {
  const uint32_t ub = (d.rank + 7) / 8;
  float c = 0.f;
#pragma unroll
  for (uint32_t p = 0; p < kUAheadPaths; ++p) {
    if (p < d.n_paths) {
      const uint64_t w = u.w[p] >> u.sh;
      for (uint32_t b = 0; b < ub; ++b) {
        const uint32_t byte = (uint32_t)(w >> (8 * b)) & 255u;
        if constexpr (DIRECT) {
          const float* z = e.z + p * d.rank + 8 * b;
          float sum = 0.f;
          for (uint32_t k = 0; k < 8 && 8 * b + k < d.rank; ++k) sum += ((byte >> k) & 1u) ? -z[k] : z[k];
          c += sum;
        } else {
          c += e.tbl[(p * ub + b) * 256 + byte];
        }
      }
    }
  }
  return c;
}

// Low-rank term of one row from the byte tables.
__device__ __forceinline__ float lowrank_row(const MatDev& d, const SegEnd& e, __amdgpu_buffer_rsrc_t ru, uint32_t row) {
  const uint32_t ub = (d.rank + 7) / 8, u0 = (uint32_t)(d.U - d.codes);
  float c = 0.f;
  for (uint32_t p = 0; p < d.n_paths; ++p)
    for (uint32_t b = 0; b < ub; ++b) {
      const uint32_t u = __builtin_amdgcn_raw_buffer_load_b8(ru, u0 + p * d.pstride + row * ub + b, 0, 0);
      c += e.tbl[(p * ub + b) * 256 + u];
    }
  return c;
}

// Stores the segment: y = ybuf (+ the low-rank term when the matrix has
// paths).  With P (a split product: this workgroup computed one pass of the
// rows, row0 a multiple of 16), the partial sums go to P[pass] instead, and
// each 16-row group of the segment counts one arrival in cnt[row / 16]; the
// workgroup whose arrival completes a group (npass arrivals) adds its rows'
// npass planes in pass order with the low-rank term, stores y, and returns
// the counter to zero.  Every thread calls it (barriers).
// With `count` (the workgroup's last segment), a segment that reads the
// low-rank terms counts the workgroup finished (finish_launch) right after
// that read, its last use of the call's tags, so that the count's round
// trip overlaps the rest of the epilogue; the last wave counts, as the
// first rows of a short segment belong to the first waves.  Returns whether
// it counted.
template <int XT, class ZJ, bool ROT>
__device__ __forceinline__ bool store_segment(const MatDev& d, uint32_t row0, uint32_t row1, const SegEnd& e,
                                              const Fuse& f, float* P = nullptr, uint32_t pass = 0,
                                              uint32_t npass = 1, uint32_t* cnt = nullptr, bool count = false) {
  __syncthreads();   // the segment's y is complete; the site table's readers are done
  const uint32_t nrows = row1 - row0;
  const __amdgpu_buffer_rsrc_t ru = rsrc(d.codes, d.blob_bytes);
  // groups of 16 rows whose last arrival this workgroup made (split only;
  // ybuf is free once the partial sums are stored)
  uint32_t* mine = reinterpret_cast<uint32_t*>(e.ybuf);
  if (P) {
    for (uint32_t i = threadIdx.x; i < nrows; i += blockDim.x) store_dev(P + (size_t)pass * d.out + row0 + i, e.ybuf[i]);
    wait_stores();   // each wave's partial sums, before the counts
    __shared__ uint32_t s_any;
    if (threadIdx.x == 0) s_any = 0;
    __syncthreads();
    const uint32_t g0 = row0 / 16, ng = (nrows + 15) / 16;
    for (uint32_t t = threadIdx.x; t < ng; t += blockDim.x) {
      const uint32_t arrived = __hip_atomic_fetch_add(cnt + g0 + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = arrived + 1 == npass;
      if (last) {
        __hip_atomic_store(cnt + g0 + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_any = 1;
      }
      mine[t] = last;
    }
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(s_any)) return false;   // no group completed here
    if (!d.terms) {
      for (uint32_t i = threadIdx.x; i < nrows; i += blockDim.x) {
        if (!mine[i / 16]) continue;
        const uint32_t row = row0 + i;
        float v = load_dev(P + row);
        for (uint32_t q = 1; q < npass; ++q) v += load_dev(P + (size_t)q * d.out + row);
        d.y[row] = v;
      }
      return false;
    }
  } else if (!d.terms) {
    for (uint32_t i = threadIdx.x; i < nrows; i += blockDim.x) d.y[row0 + i] = e.ybuf[i];
    return false;
  }
  // The low-rank term.  Every thread's U bytes for its first row go out
  // before the partials are read, so their latencies overlap.  A segment of
  // at most one row per thread needs no tables: each row's term comes
  // straight from z.
  const bool ahead = u_ahead_fits(d);
  const uint32_t i0 = threadIdx.x;
  const uint32_t urow = row0 + min(i0, nrows - 1);
  const UAhead ua = load_u_ahead(d, ru, urow);
  // A split product's completing workgroup also loads its thread's row's
  // partial sums (up to kPAhead passes) before the read, for the same reason.
  constexpr uint32_t kPAhead = 4;
  const bool direct = ahead && nrows <= blockDim.x;
  float pa[kPAhead];
#pragma unroll
  for (uint32_t q = 0; q < kPAhead; ++q) pa[q] = 0.f;
  if (P && direct && npass <= kPAhead && i0 < nrows && mine[i0 / 16]) {
#pragma unroll
    for (uint32_t q = 0; q < kPAhead; ++q)
      if (q < npass) pa[q] = load_dev(P + (size_t)q * d.out + row0 + i0);
  }
  if (!lowrank_z_read(d, e, f)) lowrank_z_here<XT, ROT>(d, e);   // the rare fallback
  __syncthreads();
  if (count) finish_launch(f, blockDim.x - 64);
  if (direct) {
    if (i0 < nrows) {
      const uint32_t row = row0 + i0;
      float v;
      if (P) {
        if (!mine[i0 / 16]) return count;
        if (npass <= kPAhead) {
          v = pa[0];
#pragma unroll
          for (uint32_t q = 1; q < kPAhead; ++q)
            if (q < npass) v += pa[q];
        } else {
          v = load_dev(P + row);
          for (uint32_t q = 1; q < npass; ++q) v += load_dev(P + (size_t)q * d.out + row);
        }
      } else {
        v = e.ybuf[i0];
      }
      d.y[row] = v + lowrank_row_ahead<true>(d, e, ua);
    }
    return count;
  }
  lowrank_build(d, e);
  for (uint32_t i = i0; i < nrows; i += blockDim.x) {
    const uint32_t row = row0 + i;
    float v;
    if (P) {
      if (!mine[i / 16]) continue;
      v = load_dev(P + row);
      for (uint32_t q = 1; q < npass; ++q) v += load_dev(P + (size_t)q * d.out + row);
    } else {
      v = e.ybuf[i];
    }
    d.y[row] = v + (ahead && i == i0 ? lowrank_row_ahead<false>(d, e, ua) : lowrank_row(d, e, ru, row));
  }
  return count;
}

}  // namespace
