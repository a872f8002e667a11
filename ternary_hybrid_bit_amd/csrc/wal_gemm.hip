// Small-batch kernels of libwal for gfx950: Y = X W^T for a batch of up to 32
// bf16 activation rows (multi-sequence decode, short prefill) on the 2-bit
// planes.  With B activation columns every decoded trit feeds B products:
//     Y[n][row] = sum_g ( alpha[row][g] * sum_{k in g} T[row][k] X[n][k]
//                       +  beta[row][g] * sum_{k in g} R[row][k] X[n][k] )
//               + sum_t (-1)^{U bit} z[n][t]
// (WAL pages, "Format": the ternary-hybrid product and its binary low-rank
// paths; the per-(row, group) scales are applied in fp32 in both kernels).
//
// Two kernels, both writing per-K-slice partial sums to the workspace, which
// a last kernel adds in a fixed order together with the low-rank term:
//  * k_gemv_batch (vector ALUs): a wavefront takes kGemvRows rows of one
//    4096-column pass for up to kGemvCols columns.  Each lane decodes its 64
//    trits of a row once (shift and mask to bf16 +-2 / 0, as the batch-1
//    kernels do) and feeds them to one v_dot2_f32_bf16 per trit pair and
//    column; the sites gather 2x from a per-pass LDS copy of X.
//  * k_mfma (matrix cores): v_mfma_f32_16x16x32_bf16 over 16 rows x 16 batch
//    columns x 32 columns of a group.  A lane (row i = lane & 15, K block
//    kb = lane >> 4) decodes its 8 code bytes straight into A operands; the
//    group's sites are scattered as +-2 into a per-wavefront LDS tile in
//    operand order, read back as a second A operand and cleared; X comes in
//    operand order from a pre-pass (k_xperm).  The two group sums land in
//    separate accumulators that alpha and beta scale in fp32.
// Decoded values are exact in bf16, the products and sums are fp32, so
// x = e_j still gives column j of W exactly.
#include <hip/hip_runtime.h>

#include "wal_device.h"
#include "wal_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// Low-rank reductions for every batch column: z[n][t], blockIdx.y = n.
__global__ __launch_bounds__(kThreads) void k_z_batch(MatDev d) {
  MatDev e = d;
  e.x = reinterpret_cast<const uint16_t*>(d.x) + (size_t)blockIdx.y * d.ldx;
  e.z = d.z + (size_t)blockIdx.y * d.terms;
  z_chunk<WAL_X_BF16, kZTerms>(e, e.x, blockIdx.x * kZTerms, e.z);
}

// Y[n][row] = sum over K slices of the partials (in slice order) + the
// low-rank term.
__global__ __launch_bounds__(256) void k_partial_reduce(MatDev d, const float* __restrict__ P, uint32_t slices) {
  const uint32_t row = blockIdx.x * 256 + threadIdx.x, n = blockIdx.y;
  if (row >= d.out) return;
  const size_t plane = (size_t)d.batch * d.out;
  float v = 0.f;
  for (uint32_t s = 0; s < slices; ++s) v += P[s * plane + (size_t)n * d.out + row];
  const uint32_t ub = (d.rank + 7) / 8;
  for (uint32_t t = 0; t < d.terms; ++t) {
    const uint32_t p = t / d.rank, r = t % d.rank;
    const uint32_t bit = (path_ptr(d.U, p)[(size_t)row * ub + r / 8] >> (r & 7)) & 1u;
    const float zt = d.z[(size_t)n * d.terms + t];
    v += bit ? -zt : zt;
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

template <int SF, int K, int NB>
__global__ __launch_bounds__(kThreads) void k_gemv_batch(MatDev d, float* __restrict__ P) {
  // X of the pass, doubled, as [column][NB] bf16: the site gathers
  __shared__ uint16_t tbl[kPass2bit * NB];
  constexpr uint32_t R = kGemvRows * NB;
  constexpr uint32_t SB = SF == WAL_SCALE_FP16 ? 2 : 3;
  const uint32_t pass = blockIdx.x, c0 = blockIdx.z * NB;
  const uint32_t col0 = pass * kPass2bit, pw = min(kPass2bit, d.in - col0);
  const int lane = threadIdx.x & 63;
  const uint16_t* X = reinterpret_cast<const uint16_t*>(d.x);

  for (uint32_t e = threadIdx.x; e < kPass2bit; e += kThreads)
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      uint32_t v = 0;
      if (e < pw && c0 + n < d.batch) v = X[(size_t)(c0 + n) * d.ldx + col0 + e];
      tbl[e * NB + n] = (uint16_t)(__float_as_uint(2.0f * __uint_as_float(v << 16)) >> 16);
    }

  const bool active = (uint32_t)lane * 64 < pw;
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
  __syncthreads();

  const uint32_t row_base = blockIdx.y * (kWaves * kGemvRows) + wave_id() * kGemvRows;
  if (row_base >= d.out) return;   // no barrier follows
  // Lanes past the pass width read their row's last group (in bounds; their
  // x pairs and scales are zero).
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

// X in operand order: Xp[g][t][m][lane][q] (bf16 pairs).  For n-tile t,
// MFMA m of group g and lane (n, kb), pair q holds X[16t + n][K_lo],
// X[16t + n][K_lo + 8] with o = 4m + q, K_lo = 128g + 32kb + 16(o >> 3) + (o & 7):
// the trit pair the A-operand decode puts in the same slot.
__global__ __launch_bounds__(256) void k_xperm(MatDev d, uint32_t nt, uint32_t* __restrict__ Xp) {
  const uint32_t id = blockIdx.x * 256 + threadIdx.x;   // (g, t, m, lane)
  if (id >= d.groups * nt * 4 * 64) return;
  const uint32_t lane = id & 63, m = (id >> 6) & 3, rest = id >> 8;
  const uint32_t t = rest % nt, g = rest / nt;
  const uint32_t n = 16 * t + (lane & 15), kb = lane >> 4;
  const uint16_t* X = reinterpret_cast<const uint16_t*>(d.x) + (size_t)n * d.ldx;
  uint32_t v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t o = 4 * m + q;
    const uint32_t klo = 128 * g + 32 * kb + 16 * (o >> 3) + (o & 7);
    v[q] = n < d.batch ? (uint32_t)X[klo] | ((uint32_t)X[klo + 8] << 16) : 0u;
  }
  reinterpret_cast<uint4*>(Xp)[id] = make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ f32x4_t mfma(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// One wavefront: kMfmaTiles row tiles x NT n-tiles over groups [g0, g1) of
// K slice ks; writes 0.5 x its partial (decoded values are 2x).
template <int SF, int K, int NT>
__global__ __launch_bounds__(kThreads) void k_mfma(MatDev d, const uint32_t* __restrict__ Xp,
                                                   float* __restrict__ P, uint32_t ks_count) {
  __shared__ uint4 rtile[kWaves][64][4];   // per-wavefront R operands, operand order
  const int lane = threadIdx.x & 63;
  const uint32_t wave = wave_id();
  const uint32_t w = blockIdx.x * kWaves + wave;
  const uint32_t rb = w / ks_count, ks = w % ks_count;
  const uint32_t row_base = rb * kMfmaRows;
  if (row_base >= d.out) return;   // whole wavefront; no barrier follows
  const uint32_t G = d.groups;
  const uint32_t g0 = (uint32_t)((uint64_t)ks * G / ks_count);
  const uint32_t g1 = (uint32_t)((uint64_t)(ks + 1) * G / ks_count);
  constexpr uint32_t SB = SF == WAL_SCALE_FP16 ? 2 : 3;
  const uint32_t i = lane & 15, kb = lane >> 4;
  uint4* rt = rtile[wave][0];
  uint16_t* rt16 = reinterpret_cast<uint16_t*>(rtile[wave][0]);
  if constexpr (K > 0) {
#pragma unroll
    for (int m = 0; m < 4; ++m) rt[lane * 4 + m] = make_uint4(0, 0, 0, 0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  }

  const __amdgpu_buffer_rsrc_t rc = rsrc(d.codes, d.blob_bytes);
  const __amdgpu_buffer_rsrc_t ra = rsrc(d.alpha, d.blob_bytes - (uint32_t)(d.alpha - d.codes));
  __amdgpu_buffer_rsrc_t rs = rsrc(d.codes, 0u), rbe = rsrc(d.codes, 0u);
  if constexpr (K > 0) {
    rs = rsrc(d.sites, d.blob_bytes - (uint32_t)(d.sites - d.codes));
    rbe = rsrc(d.beta, d.blob_bytes - (uint32_t)(d.beta - d.codes));
  }
  // lanes 0-15 fetch alpha of tile row (lane & 15), lanes 16-31 its beta
  const bool fetch_beta = K > 0 && lane >= 16;

  f32x4_t C[kMfmaTiles][NT];
#pragma unroll
  for (uint32_t r = 0; r < kMfmaTiles; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) C[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (uint32_t g = g0; g < g1; ++g) {
    uint4 xb[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        xb[t][m] = reinterpret_cast<const uint4*>(Xp)[(((size_t)g * NT + t) * 4 + m) * 64 + lane];
#pragma unroll
    for (uint32_t r = 0; r < kMfmaTiles; ++r) {
      const uint32_t row = min(row_base + 16 * r + i, d.out - 1);
      const u32x2_t c = __builtin_bit_cast(
          u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rc, g * 32 + 8 * kb, row * d.row_stride, kStream));
      const uint32_t sraw = fetch_beta ? load_scale<SF>(rbe, g * SB, row * G * SB)
                                       : load_scale<SF>(ra, g * SB, row * G * SB);
      uint4 a[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t op[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int o = 4 * m + q;
          op[q] = (c[o >> 3] << (14 - 2 * (o & 7))) & 0xC000C000u;
        }
        a[m] = make_uint4(op[0], op[1], op[2], op[3]);
      }
      f32x4_t sT[NT], sR[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        sT[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) sT[t] = mfma(a[m], xb[t][m], sT[t]);
      }
      if constexpr (K > 0) {
        // lane (i, kb) scatters sites kb * K / 4 .. of row i (K = 2: the
        // lanes with kb < 2, one site each)
        uint32_t sbytes;
        if constexpr (K == 8) sbytes = __builtin_amdgcn_raw_buffer_load_b16(rs, g * 8 + 2 * kb, row * G * 8, kStream);
        else if constexpr (K == 4) sbytes = __builtin_amdgcn_raw_buffer_load_b8(rs, g * 4 + kb, row * G * 4, kStream);
        else sbytes = __builtin_amdgcn_raw_buffer_load_b8(rs, g * 2 + (kb & 1), row * G * 2, kStream);
        constexpr int PER = K == 8 ? 2 : 1;
        const bool writer = K != 2 || kb < 2;
        uint32_t addr[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const uint32_t sb = (sbytes >> (8 * j)) & 0xFFu;
          const uint32_t pos = sb & 127u, local = pos & 31u, rr = local & 15u;
          const uint32_t o = 8 * (local >> 4) + (rr & 7u);
          const uint32_t lt = (pos >> 5) * 16 + i;   // lane whose operand holds column pos of row i
          addr[j] = lt * 32 + (o >> 2) * 8 + (o & 3) * 2 + (rr >> 3);
          if (writer) rt16[addr[j]] = (sb & 128u) ? 0xC000u : 0x4000u;
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        uint4 ro[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) ro[m] = rt[lane * 4 + m];
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
        for (int j = 0; j < PER; ++j)
          if (writer) rt16[addr[j]] = 0;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          sR[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < 4; ++m) sR[t] = mfma(ro[m], xb[t][m], sR[t]);
        }
      }
      // C layout: lane holds rows 4 kb + j of the tile, batch column i
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int src = 4 * kb + j;
        const float al = scale_value<SF>((uint32_t)__builtin_amdgcn_ds_bpermute(4 * src, (int)sraw));
#pragma unroll
        for (int t = 0; t < NT; ++t) C[r][t][j] = __builtin_fmaf(al, sT[t][j], C[r][t][j]);
        if constexpr (K > 0) {
          const float be = scale_value<SF>((uint32_t)__builtin_amdgcn_ds_bpermute(4 * (16 + src), (int)sraw));
#pragma unroll
          for (int t = 0; t < NT; ++t) C[r][t][j] = __builtin_fmaf(be, sR[t][j], C[r][t][j]);
        }
      }
    }
  }
#pragma unroll
  for (uint32_t r = 0; r < kMfmaTiles; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t n = 16 * t + i;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t row = row_base + 16 * r + 4 * kb + j;
        if (n < d.batch && row < d.out) P[((size_t)ks * d.batch + n) * d.out + row] = 0.5f * C[r][t][j];
      }
    }
}

// ---------------------------------------------------------------------------
// Host side.

uint32_t class_index(const MatDev& d) {
  return d.scale_fmt * 4 + (d.k == 0 ? 0 : d.k == 2 ? 1 : d.k == 4 ? 2 : 3);
}

template <int SF, int K>
void launch_gemv_nb(uint32_t nb, dim3 grid, hipStream_t s, const MatDev& d, float* P) {
  if (nb == 1) hipLaunchKernelGGL((k_gemv_batch<SF, K, 1>), grid, dim3(kThreads), 0, s, d, P);
  else if (nb == 2) hipLaunchKernelGGL((k_gemv_batch<SF, K, 2>), grid, dim3(kThreads), 0, s, d, P);
  else hipLaunchKernelGGL((k_gemv_batch<SF, K, 4>), grid, dim3(kThreads), 0, s, d, P);
}

template <int SF, int K>
void launch_mfma_nt(uint32_t nt, dim3 grid, hipStream_t s, const MatDev& d, const uint32_t* Xp, float* P,
                    uint32_t ks) {
  if (nt == 1) hipLaunchKernelGGL((k_mfma<SF, K, 1>), grid, dim3(kThreads), 0, s, d, Xp, P, ks);
  else hipLaunchKernelGGL((k_mfma<SF, K, 2>), grid, dim3(kThreads), 0, s, d, Xp, P, ks);
}

// z pre-pass into the workspace; points the descriptor at it.
bool launch_z(MatDev& d, const GemmShape& S, uint8_t* ws, uint32_t batch, hipStream_t s) {
  d.z = reinterpret_cast<float*>(ws + S.off_z);
  if (!d.terms) return true;
  hipLaunchKernelGGL(k_z_batch, dim3((d.terms + kZTerms - 1) / kZTerms, batch), dim3(kThreads), 0, s, d);
  return hipGetLastError() == hipSuccess;
}

}  // namespace

namespace wal {

int launch_gemm_valu(const wal_info& f, const MatDev& d0, uint32_t batch, void* ws, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const GemmShape S = gemm_shape(f, batch);
  uint8_t* w = static_cast<uint8_t*>(ws);
  MatDev d = d0;
  if (!launch_z(d, S, w, batch, s)) return WAL_ERR_DEVICE;
  float* P = reinterpret_cast<float*>(w + S.off_p);
  const uint32_t nb = batch >= 3 ? kGemvCols : batch;
  const dim3 grid(S.passes, (f.d.out + kWaves * kGemvRows - 1) / (kWaves * kGemvRows), (batch + nb - 1) / nb);
  switch (class_index(d)) {
    case 0: launch_gemv_nb<WAL_SCALE_FP16, 0>(nb, grid, s, d, P); break;
    case 1: launch_gemv_nb<WAL_SCALE_FP16, 2>(nb, grid, s, d, P); break;
    case 2: launch_gemv_nb<WAL_SCALE_FP16, 4>(nb, grid, s, d, P); break;
    case 3: launch_gemv_nb<WAL_SCALE_FP16, 8>(nb, grid, s, d, P); break;
    case 4: launch_gemv_nb<WAL_SCALE_FP24, 0>(nb, grid, s, d, P); break;
    case 5: launch_gemv_nb<WAL_SCALE_FP24, 2>(nb, grid, s, d, P); break;
    case 6: launch_gemv_nb<WAL_SCALE_FP24, 4>(nb, grid, s, d, P); break;
    default: launch_gemv_nb<WAL_SCALE_FP24, 8>(nb, grid, s, d, P); break;
  }
  if (hipGetLastError() != hipSuccess) return WAL_ERR_DEVICE;
  hipLaunchKernelGGL(k_partial_reduce, dim3((f.d.out + 255) / 256, batch), dim3(256), 0, s, d, P, S.passes);
  return hipGetLastError() == hipSuccess ? WAL_OK : WAL_ERR_DEVICE;
}

int launch_gemm_mfma(const wal_info& f, const MatDev& d0, uint32_t batch, void* ws, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const GemmShape S = gemm_shape(f, batch);
  uint8_t* w = static_cast<uint8_t*>(ws);
  MatDev d = d0;
  if (!launch_z(d, S, w, batch, s)) return WAL_ERR_DEVICE;
  uint32_t* Xp = reinterpret_cast<uint32_t*>(w + S.off_xp);
  float* P = reinterpret_cast<float*>(w + S.off_p);
  const uint32_t nx = f.groups * S.nt * 4 * 64;
  hipLaunchKernelGGL(k_xperm, dim3((nx + 255) / 256), dim3(256), 0, s, d, S.nt, Xp);
  if (hipGetLastError() != hipSuccess) return WAL_ERR_DEVICE;
  const dim3 grid((S.row_blocks * S.ks + kWaves - 1) / kWaves);
  switch (class_index(d)) {
    case 0: launch_mfma_nt<WAL_SCALE_FP16, 0>(S.nt, grid, s, d, Xp, P, S.ks); break;
    case 1: launch_mfma_nt<WAL_SCALE_FP16, 2>(S.nt, grid, s, d, Xp, P, S.ks); break;
    case 2: launch_mfma_nt<WAL_SCALE_FP16, 4>(S.nt, grid, s, d, Xp, P, S.ks); break;
    case 3: launch_mfma_nt<WAL_SCALE_FP16, 8>(S.nt, grid, s, d, Xp, P, S.ks); break;
    case 4: launch_mfma_nt<WAL_SCALE_FP24, 0>(S.nt, grid, s, d, Xp, P, S.ks); break;
    case 5: launch_mfma_nt<WAL_SCALE_FP24, 2>(S.nt, grid, s, d, Xp, P, S.ks); break;
    case 6: launch_mfma_nt<WAL_SCALE_FP24, 4>(S.nt, grid, s, d, Xp, P, S.ks); break;
    default: launch_mfma_nt<WAL_SCALE_FP24, 8>(S.nt, grid, s, d, Xp, P, S.ks); break;
  }
  if (hipGetLastError() != hipSuccess) return WAL_ERR_DEVICE;
  hipLaunchKernelGGL(k_partial_reduce, dim3((f.d.out + 255) / 256, batch), dim3(256), 0, s, d, P, S.ks);
  return hipGetLastError() == hipSuccess ? WAL_OK : WAL_ERR_DEVICE;
}

}  // namespace wal
