// Normalised Hadamard-128 rotation of activations for gfx950:
//     out[r][128 g + i] = sum_j H[i][j] x[r][128 g + j] / sqrt(128)
// with H Sylvester's 128 x 128 Hadamard matrix, H[i][j] = (-1)^popcount(i & j)
// (WAL2-Ternary-27B card, "Архитектура": its packed weights are rotated by a
// normalised H128 with sign_mode identity, so a product of such a blob takes
// the rotated activations; the weight side is unchanged).
//
// Eight lanes take one 128-column group, 16 consecutive values each.  The
// butterflies (a, b) -> (a + b, a - b) over index bits 0..3 run inside a lane,
// those over bits 4..6 between the eight lanes (xor shuffles); all in fp32,
// then one multiply by 1/sqrt(128) and a round to nearest even into the
// output type.  A lane reads its 16 values before it writes them, and lanes
// exchange values only through registers, so the rotation may run in place.
#include <hip/hip_runtime.h>

#include "wal_internal.h"

namespace {

constexpr float kInvSqrt128 = 0.08838834764831845f;   // 1 / sqrt(128), rounded to fp32

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;   // NaN stays NaN
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int XT, int OT>
__global__ __launch_bounds__(256) void k_rotate_h128(const void* __restrict__ x, uint32_t ldx, void* out,
                                                     uint32_t ldo, uint32_t rows, uint32_t groups) {
  const uint32_t t = blockIdx.x * 256 + threadIdx.x;
  const uint32_t gid = t >> 3, sub = t & 7;
  const bool valid = gid < rows * groups;   // the same for the 8 lanes of a group
  const uint32_t r = valid ? gid / groups : 0, g = valid ? gid % groups : 0;
  const uint32_t c0 = 128 * g + 16 * sub;
  float v[16];
  if constexpr (XT == WAL_X_BF16) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + (size_t)r * ldx + c0);
    const uint4 a = valid ? src[0] : make_uint4(0, 0, 0, 0), b = valid ? src[1] : make_uint4(0, 0, 0, 0);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(x) + (size_t)r * ldx + c0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 a = valid ? src[k] : make_float4(0.f, 0.f, 0.f, 0.f);
      v[4 * k] = a.x; v[4 * k + 1] = a.y; v[4 * k + 2] = a.z; v[4 * k + 3] = a.w;
    }
  }
  // index bits 0..3: inside the lane
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (!(j & h)) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
  // index bits 4..6: lane bits 0..2 of the group's eight lanes; the lane with
  // the bit set holds the second element of each pair
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) {
    const bool second = sub & m;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float p = __shfl_xor(v[j], m);
      v[j] = second ? p - v[j] : v[j] + p;
    }
  }
  if (!valid) return;
  if constexpr (OT == WAL_X_BF16) {
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = bf16_rne(v[2 * k] * kInvSqrt128) | (bf16_rne(v[2 * k + 1] * kInvSqrt128) << 16);
    uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + (size_t)r * ldo + c0);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + (size_t)r * ldo + c0);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      dst[k] = make_float4(v[4 * k] * kInvSqrt128, v[4 * k + 1] * kInvSqrt128, v[4 * k + 2] * kInvSqrt128,
                           v[4 * k + 3] * kInvSqrt128);
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int wal_rotate_h128(const void* x_dev, int x_dtype, uint32_t rows, uint32_t in, uint32_t ldx,
                               void* out_dev, int out_dtype, uint32_t ldo, void* stream) {
  if (!x_dev || !out_dev || !rows) return WAL_ERR_ARG;
  if (x_dtype != WAL_X_F32 && x_dtype != WAL_X_BF16) return WAL_ERR_ARG;
  if (out_dtype != WAL_X_F32 && out_dtype != WAL_X_BF16) return WAL_ERR_ARG;
  if (in == 0 || in % 128) return WAL_ERR_SHAPE;
  if (ldx < in || ldo < in) return WAL_ERR_ARG;
  const size_t xe = x_dtype == WAL_X_BF16 ? 2 : 4, oe = out_dtype == WAL_X_BF16 ? 2 : 4;
  if (!aligned16(x_dev) || !aligned16(out_dev) || (ldx * xe) % 16 || (ldo * oe) % 16) return WAL_ERR_ALIGN;
  const uint64_t groups = in / 128, total = (uint64_t)rows * groups;
  if (total >= (1ull << 28)) return WAL_ERR_SHAPE;
  // in place only exactly (same buffer, type and pitch); other overlaps are rejected
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x_dev), oa = reinterpret_cast<uintptr_t>(out_dev);
  const uint64_t xb = ((uint64_t)(rows - 1) * ldx + in) * xe, ob = ((uint64_t)(rows - 1) * ldo + in) * oe;
  const bool same = xa == oa && x_dtype == out_dtype && ldx == ldo;
  if (!same && xa < oa + ob && oa < xa + xb) return WAL_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((uint32_t)((total * 8 + 255) / 256));
  if (x_dtype == WAL_X_BF16 && out_dtype == WAL_X_BF16)
    hipLaunchKernelGGL((k_rotate_h128<WAL_X_BF16, WAL_X_BF16>), grid, dim3(256), 0, s, x_dev, ldx, out_dev, ldo, rows, (uint32_t)groups);
  else if (x_dtype == WAL_X_BF16)
    hipLaunchKernelGGL((k_rotate_h128<WAL_X_BF16, WAL_X_F32>), grid, dim3(256), 0, s, x_dev, ldx, out_dev, ldo, rows, (uint32_t)groups);
  else if (out_dtype == WAL_X_BF16)
    hipLaunchKernelGGL((k_rotate_h128<WAL_X_F32, WAL_X_BF16>), grid, dim3(256), 0, s, x_dev, ldx, out_dev, ldo, rows, (uint32_t)groups);
  else
    hipLaunchKernelGGL((k_rotate_h128<WAL_X_F32, WAL_X_F32>), grid, dim3(256), 0, s, x_dev, ldx, out_dev, ldo, rows, (uint32_t)groups);
  return hipGetLastError() == hipSuccess ? WAL_OK : WAL_ERR_DEVICE;
}
