// Normalised Hadamard-128 rotation of activations for gfx950:
//     out[r][128 g + i] = sum_j H[i][j] x[r][128 g + j] / sqrt(128)
// with H Sylvester's 128 x 128 Hadamard matrix, H[i][j] = (-1)^popcount(i & j)
// (WAL2-Ternary-27B card, "Архитектура": its packed weights are rotated by a
// normalised H128 with sign_mode identity, so a product of such a blob takes
// the rotated activations; the weight side is unchanged).
//
// The arithmetic is the one the products use when they rotate x themselves
// (wal_device.h), so rotating here and multiplying gives the same bits:
//  * bf16 input: a workgroup takes up to 32 consecutive groups of one row as
//    the product X H on the matrix cores (v_mfma_f32_16x16x32_bf16, exact
//    bf16 operands, fp32 sums), scales by fp32(1/sqrt(128)) and rounds to
//    nearest even for bf16 output (v_cvt_pk_bf16_f32).
//  * fp32 input: eight lanes take one group, 16 consecutive values each; the
//    butterflies (a, b) -> (a + b, a - b) over index bits 0..3 run inside a
//    lane, those over bits 4..6 between the eight lanes (xor shuffles), all
//    in fp32, then the scale and, for bf16 output, a round to nearest even.
// Every workgroup reads all its inputs before any of its lanes writes, and
// groups never straddle workgroups, so the rotation may run in place.
// (rows x ceil(in / 4096) workgroups with bf16 input: below 2^28 groups the
// count fits a grid.)
#include <hip/hip_runtime.h>

#include "wal_device.h"
#include "wal_internal.h"

namespace {

// bf16 input: a workgroup takes 32 consecutive groups of one row (chunk
// blockIdx.x % chunks of row blockIdx.x / chunks) on the matrix cores.
template <int OT>
__global__ __launch_bounds__(256) void k_rotate_h128_mfma(const uint16_t* __restrict__ x, uint32_t ldx, void* out,
                                                          uint32_t ldo, uint32_t groups, uint32_t chunks) {
  const uint32_t row = blockIdx.x / chunks, g0 = 32 * (blockIdx.x % chunks);
  const uint32_t ng = min(32u, groups - g0);
  const __amdgpu_buffer_rsrc_t rx = rsrc(x + (size_t)row * ldx + 128 * g0, 256 * ng);
  RotTiles<2, OT == WAL_X_F32> t;
  t.load(rx, 0, ng);
  t.compute();
  __syncthreads();   // every wave has read its inputs (in-place rotation)
#pragma unroll
  for (int gt = 0; gt < 2; ++gt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t g = t.group(gt, jj);
      if (g >= ng) continue;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const size_t e = (size_t)row * ldo + 128 * (g0 + g) + t.column(u);
        if constexpr (OT == WAL_X_BF16)
          static_cast<uint16_t*>(out)[e] = (uint16_t)t.bits(gt, u, jj);
        else
          static_cast<float*>(out)[e] = t.f[gt][u][jj];
      }
    }
}

// fp32 input: eight lanes per group, 16 values each.
template <int OT>
__global__ __launch_bounds__(256) void k_rotate_h128_f32(const float* __restrict__ x, uint32_t ldx, void* out,
                                                         uint32_t ldo, uint32_t rows, uint32_t groups) {
  const uint32_t t = blockIdx.x * 256 + threadIdx.x;
  const uint32_t gid = t >> 3, sub = t & 7;
  const bool valid = gid < rows * groups;   // the same for the 8 lanes of a group
  const uint32_t r = valid ? gid / groups : 0, g = valid ? gid % groups : 0;
  const uint32_t c0 = 128 * g + 16 * sub;
  float v[16];
  const float4* src = reinterpret_cast<const float4*>(x + (size_t)r * ldx + c0);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 a = valid ? src[k] : make_float4(0.f, 0.f, 0.f, 0.f);
    v[4 * k] = a.x; v[4 * k + 1] = a.y; v[4 * k + 2] = a.z; v[4 * k + 3] = a.w;
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
  const uint32_t chunks = (uint32_t)((groups + 31) / 32);
  const dim3 grid((uint32_t)((total + 31) / 32)), grid_rows(rows * chunks);   // 32 groups per workgroup
  const uint16_t* xh = static_cast<const uint16_t*>(x_dev);
  const float* xf = static_cast<const float*>(x_dev);
  if (x_dtype == WAL_X_BF16 && out_dtype == WAL_X_BF16)
    hipLaunchKernelGGL(k_rotate_h128_mfma<WAL_X_BF16>, grid_rows, dim3(256), 0, s, xh, ldx, out_dev, ldo, (uint32_t)groups, chunks);
  else if (x_dtype == WAL_X_BF16)
    hipLaunchKernelGGL(k_rotate_h128_mfma<WAL_X_F32>, grid_rows, dim3(256), 0, s, xh, ldx, out_dev, ldo, (uint32_t)groups, chunks);
  else if (out_dtype == WAL_X_BF16)
    hipLaunchKernelGGL(k_rotate_h128_f32<WAL_X_BF16>, grid, dim3(256), 0, s, xf, ldx, out_dev, ldo, rows, (uint32_t)groups);
  else
    hipLaunchKernelGGL(k_rotate_h128_f32<WAL_X_F32>, grid, dim3(256), 0, s, xf, ldx, out_dev, ldo, rows, (uint32_t)groups);
  return hipGetLastError() == hipSuccess ? WAL_OK : WAL_ERR_DEVICE;
}
