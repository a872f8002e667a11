// gfx950 (CDNA4) kernels and the product entry points of libwal.
//
// Operator (WAL-Ternary-8B cards, "Модель пішімі" / "Representation"):
//     y = (alpha * T + beta * R) x + sum_p U_p diag(s_p) V_p^T x
// computed straight from the packed planes described in include/wal.h.
//
// Kernel design (one 64-wide wavefront streams whole rows):
//  * Codes.  Each lane owns 64 consecutive columns of a 4096-column pass and
//    loads its 16 bytes of 2-bit codes per row with one 128-bit load, so a
//    wavefront reads a 1 KB row segment fully coalesced.  A code keeps its
//    magnitude bit below its sign bit, so shifting a code pair to bits 14-15
//    and 30-31 and masking with 0xC000C000 yields a packed bf16 pair whose
//    halves are +-2.0 or 0: the trits become sign-selected copies of x with
//    no multiply and no table.  v_dot2c_f32_bf16 then adds both halves into
//    an fp32 accumulator (products by +-2 and 0 are exact).  The lane's x
//    stays in registers for the whole pass, pre-arranged in the same pairs.
//  * Sites.  A per-workgroup LDS table holds +x and -x for every position of
//    every group of the pass ([group][256] floats), so a site byte (7-bit
//    position, sign in bit 7) indexes its signed value directly.
//  * Scales.  alpha multiplies the lane's ternary partial and beta its site
//    partial once per row and group, in fp32 (fp16 or fp24 decoded in
//    registers).
//  * Low rank.  A pre-pass computes z = diag(s) V^T x per path and rank; in
//    the main pass lane t adds +-z[t] by the row's U bit before the row's
//    wavefront reduction (DPP adds, no LDS).
//  * Rows are reduced with DPP and their totals parked in lane (row - n0) of
//    one register, so y is stored with one coalesced write per wavefront.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <cstring>

#include "wal_internal.h"

using namespace wal;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

namespace {

constexpr uint32_t kRowsMax = 64;   // rows one wavefront parks in a register

// ---------------------------------------------------------------------------
// Wavefront reduction: four DPP steps sum each row of 16 lanes, two row
// broadcasts fold the rows into lane 63.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_term(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_term<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_term<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_term<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_term<0x140, 0xF>(v);  // row_mirror
  v += dpp_term<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_term<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// ---------------------------------------------------------------------------
// Scales: fp16, or fp24 = the upper 24 bits of an fp32 pattern.
__device__ __forceinline__ uint32_t load_scale_raw(const uint8_t* p, uint32_t sfmt) {
  if (sfmt == WAL_SCALE_FP16) return *reinterpret_cast<const uint16_t*>(p);
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16);
}
__device__ __forceinline__ float decode_scale(uint32_t raw, uint32_t sfmt) {
  if (sfmt == WAL_SCALE_FP16) return __half2float(__ushort_as_half((unsigned short)raw));
  return __uint_as_float(raw << 8);
}
__device__ __forceinline__ uint32_t scale_bytes(uint32_t sfmt) { return sfmt == WAL_SCALE_FP16 ? 2u : 3u; }

// Activation element as fp32.
template <int XT>
__device__ __forceinline__ float xval(const void* x, uint32_t i) {
  if (XT == WAL_X_F32) return reinterpret_cast<const float*>(x)[i];
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[i] << 16);
}

// ---------------------------------------------------------------------------
// A lane's 64 activation columns for one pass, held in registers.
template <int XT> struct XLane;

template <> struct XLane<WAL_X_BF16> {
  // p[8d + i] = bf16 pair (x[c + 16d + i], x[c + 16d + 8 + i]): the pair of
  // columns whose codes sit at bits 2i and 2i + 16 of the lane's dword d.
  uint32_t p[32];
  static constexpr float kScale = 0.5f;   // the decoded trits are +-2

  __device__ __forceinline__ void load(const void* x, uint32_t c, bool active) {
    if (!active) {
#pragma unroll
      for (int q = 0; q < 32; ++q) p[q] = 0;
      return;
    }
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + c);
    uint32_t w[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint4 v = src[q];
      w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int lo = 16 * d + i, hi = 16 * d + 8 + i;
        const uint32_t xl = (w[lo >> 1] >> (16 * (lo & 1))) & 0xFFFFu;
        const uint32_t xh = (w[hi >> 1] >> (16 * (hi & 1))) & 0xFFFFu;
        p[8 * d + i] = xl | (xh << 16);
      }
  }

  // 2 * sum_j T_j x_j over the lane's 64 columns of one row.
  __device__ __forceinline__ float dot(const uint4& c) const {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t op = (w[d] << (14 - 2 * i)) & 0xC000C000u;
        acc[d] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, op),
                                                 __builtin_bit_cast(bf16x2_t, p[8 * d + i]), acc[d], false);
      }
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
};

template <> struct XLane<WAL_X_F32> {
  float f[64];
  static constexpr float kScale = 1.0f;

  __device__ __forceinline__ void load(const void* x, uint32_t c, bool active) {
    if (!active) {
#pragma unroll
      for (int q = 0; q < 64; ++q) f[q] = 0.f;
      return;
    }
    const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + c);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float4 v = src[q];
      f[4 * q] = v.x; f[4 * q + 1] = v.y; f[4 * q + 2] = v.z; f[4 * q + 3] = v.w;
    }
  }

  // sum_j T_j x_j: sign-extend each 2-bit code to {-1, 0, +1} and accumulate.
  __device__ __forceinline__ float dot(const uint4& c) const {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = (int)(w[d] << (30 - 2 * i)) >> 30;
        acc[d] = __builtin_fmaf((float)t, f[16 * d + i], acc[d]);
      }
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
};

// ---------------------------------------------------------------------------
// Per-lane low-rank terms: lane t (+64 j) owns term t = p * rank + r.
struct LowRank {
  float z[4];
  const uint8_t* u[4];
  uint32_t bit[4];
  uint32_t ub;      // bytes per row of U
};

__device__ __forceinline__ void lowrank_setup(const MatDev& d, int lane, LowRank& lr) {
  lr.ub = (d.rank + 7) / 8;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t t = lane + 64 * j;
    lr.z[j] = 0.f;
    lr.u[j] = nullptr;
    lr.bit[j] = 0;
    if (t < d.terms) {
      const uint32_t p = t / d.rank, r = t % d.rank;
      lr.z[j] = d.z[t];
      lr.u[j] = d.U[p] + r / 8;
      lr.bit[j] = r % 8;
    }
  }
}

// ---------------------------------------------------------------------------
// Row data of one row and one pass, loaded ahead of its use.
struct RowData {
  uint4 c;
  uint32_t s;       // site bytes of this lane
  uint32_t a, b;    // raw alpha, beta
  uint32_t u;       // U bits of this lane's low-rank terms (bit j = term j)
};

template <int K>
struct SiteMap {
  static constexpr int SPL = K >= 4 ? 4 : K;   // sites per lane
  static constexpr int LPG = K == 8 ? 2 : 1;   // lanes per group
};

template <int XT, int K>
__device__ __forceinline__ void pass_rows_2bit(const MatDev& d, uint32_t n0, int nrows, uint32_t pass,
                                               uint32_t Gp, bool last, const float* __restrict__ tbl,
                                               const XLane<XT>& xl, const LowRank& lr, int lane,
                                               float& rowacc) {
  using SM = SiteMap<K>;
  const uint32_t G = d.groups;
  const uint32_t sb = scale_bytes(d.scale_fmt);
  const uint32_t g0 = pass * (kPass2bit / 128);
  const bool code_on = (uint32_t)lane < 2 * Gp;          // 64 columns per lane
  const uint32_t tg = lane >> 1;                          // group of the lane's codes
  const bool site_on = K > 0 && (uint32_t)lane < Gp * SM::LPG;
  const uint32_t sg = K > 0 ? lane / SM::LPG : 0;         // group of the lane's sites
  const uint32_t sofs = K > 0 ? sg * K + (lane % SM::LPG) * SM::SPL : 0;

  auto load = [&](uint32_t n) {
    RowData r;
    r.c = make_uint4(0, 0, 0, 0);
    r.s = 0; r.a = 0; r.b = 0; r.u = 0;
    if (code_on) {
      r.c = *reinterpret_cast<const uint4*>(d.codes + (size_t)n * d.row_stride + pass * (kPass2bit / 4) + 16 * lane);
      r.a = load_scale_raw(d.alpha + ((size_t)n * G + g0 + tg) * sb, d.scale_fmt);
    }
    if (K > 0 && site_on) {
      const uint8_t* sp = d.sites + ((size_t)n * G + g0) * K + sofs;
      if (SM::SPL == 4) r.s = *reinterpret_cast<const uint32_t*>(sp);
      else r.s = *reinterpret_cast<const uint16_t*>(sp);
      r.b = load_scale_raw(d.beta + ((size_t)n * G + g0 + sg) * sb, d.scale_fmt);
    }
    if (last) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lr.u[j]) r.u |= (uint32_t)((lr.u[j][(size_t)n * lr.ub] >> lr.bit[j]) & 1u) << j;
    }
    return r;
  };

  RowData cur = load(n0);
  for (int i = 0; i < nrows; ++i) {
    RowData nxt;
    if (i + 1 < nrows) nxt = load(n0 + i + 1);
    float part = 0.f;
    if (code_on) part = XLane<XT>::kScale * decode_scale(cur.a, d.scale_fmt) * xl.dot(cur.c);
    if (K > 0 && site_on) {
      float accR = 0.f;
#pragma unroll
      for (int j = 0; j < SM::SPL; ++j) accR += tbl[sg * 256 + ((cur.s >> (8 * j)) & 0xFFu)];
      part = __builtin_fmaf(decode_scale(cur.b, d.scale_fmt), accR, part);
    }
    if (last) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lr.u[j]) part += ((cur.u >> j) & 1u) ? -lr.z[j] : lr.z[j];
    }
    const float total = wave_sum(part);
    if (lane == i) rowacc += total;
    cur = nxt;
  }
}

// One tile: kWavesPerBlock wavefronts, each owning RW consecutive rows.
template <int XT>
__device__ __forceinline__ void tile_2bit(const MatDev& d, uint32_t row0, uint32_t RW, float* tbl) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t n0 = row0 + wave * RW;
  const int nrows = n0 < d.out ? (int)min(RW, d.out - n0) : 0;
  const uint32_t npass = (d.in + kPass2bit - 1) / kPass2bit;
  LowRank lr;
  lowrank_setup(d, lane, lr);
  float rowacc = 0.f;
  for (uint32_t pass = 0; pass < npass; ++pass) {
    const uint32_t pw = min(kPass2bit, d.in - pass * kPass2bit);
    const uint32_t Gp = pw / 128;
    __syncthreads();                                   // previous readers of tbl are done
    if (d.k) {
      for (uint32_t e = threadIdx.x; e < Gp * 256; e += kBlockThreads) {
        const uint32_t g = e >> 8, b = e & 255u;
        const float v = xval<XT>(d.x, pass * kPass2bit + g * 128 + (b & 127u));
        tbl[e] = (b & 128u) ? -v : v;
      }
    }
    __syncthreads();
    if (nrows > 0) {
      XLane<XT> xl;
      xl.load(d.x, pass * kPass2bit + 64 * lane, (uint32_t)(64 * lane) < pw);
      const bool last = pass + 1 == npass;
      switch (d.k) {
        case 0: pass_rows_2bit<XT, 0>(d, n0, nrows, pass, Gp, last, tbl, xl, lr, lane, rowacc); break;
        case 2: pass_rows_2bit<XT, 2>(d, n0, nrows, pass, Gp, last, tbl, xl, lr, lane, rowacc); break;
        case 4: pass_rows_2bit<XT, 4>(d, n0, nrows, pass, Gp, last, tbl, xl, lr, lane, rowacc); break;
        default: pass_rows_2bit<XT, 8>(d, n0, nrows, pass, Gp, last, tbl, xl, lr, lane, rowacc); break;
      }
    }
  }
  if (lane < nrows) d.y[n0 + lane] = rowacc;
}

template <int XT>
__global__ __launch_bounds__(kBlockThreads) void k_gemv2_single(MatDev d, uint32_t RW) {
  __shared__ float tbl[32 * 256];
  tile_2bit<XT>(d, blockIdx.x * kWavesPerBlock * RW, RW, tbl);
}

template <int XT>
__global__ __launch_bounds__(kBlockThreads) void k_gemv2_grouped(const MatDev* __restrict__ descs,
                                                                 const uint2* __restrict__ tiles,
                                                                 uint32_t n_tiles, uint32_t RW) {
  __shared__ float tbl[32 * 256];
  for (uint32_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
    const uint2 tl = tiles[t];
    tile_2bit<XT>(descs[tl.x], tl.y, RW, tbl);
  }
}

// ---------------------------------------------------------------------------
// Low-rank pre-pass: z[t] = s_p[r] * sum_j (-1)^{V_p[r] bit j} x_j, one
// wavefront per term t = p * rank + r.
template <int XT>
__device__ __forceinline__ void zjob(const MatDev& d, uint32_t t, int lane) {
  const uint32_t p = t / d.rank, r = t % d.rank;
  const uint8_t* vrow = d.V[p] + (size_t)r * (d.in / 8);
  float acc = 0.f;
  for (uint32_t c = 64 * lane; c < d.in; c += 64 * 64) {
    const uint2 bits = *reinterpret_cast<const uint2*>(vrow + c / 8);
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const float v = xval<XT>(d.x, c + j);
      const uint32_t bit = j < 32 ? (bits.x >> j) & 1u : (bits.y >> (j - 32)) & 1u;
      acc += bit ? -v : v;
    }
  }
  const float total = wave_sum(acc);
  if (lane == 0) {
    const float s = __half2float(__ushort_as_half(reinterpret_cast<const uint16_t*>(d.s[p])[r]));
    d.z[t] = s * total;
  }
}

template <int XT>
__global__ __launch_bounds__(kBlockThreads) void k_z_single(MatDev d) {
  const uint32_t t = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (t < d.terms) zjob<XT>(d, t, threadIdx.x & 63);
}

template <int XT>
__global__ __launch_bounds__(kBlockThreads) void k_z_grouped(const MatDev* __restrict__ descs,
                                                             const uint32_t* __restrict__ jobs, uint32_t n) {
  const uint32_t j = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (j < n) {
    const uint32_t job = jobs[j];
    zjob<XT>(descs[job >> 8], job & 255u, threadIdx.x & 63);
  }
}

// ---------------------------------------------------------------------------
// Host helpers.

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t xelem(int xdt) { return xdt == WAL_X_F32 ? 4 : 2; }

MatDev make_dev(const wal_info* f, const void* W, const void* x, float* y, float* z, uint32_t ldx,
                uint32_t ldy, uint32_t batch) {
  MatDev m{};
  const uint8_t* base = static_cast<const uint8_t*>(W);
  m.codes = base + f->off_codes;
  m.sites = f->d.k ? base + f->off_sites : nullptr;
  m.alpha = base + f->off_alpha;
  m.beta = f->d.k ? base + f->off_beta : nullptr;
  for (uint32_t p = 0; p < WAL_MAX_PATHS; ++p) {
    const bool on = p < f->d.n_paths;
    m.V[p] = on ? base + f->off_V[p] : nullptr;
    m.U[p] = on ? base + f->off_U[p] : nullptr;
    m.s[p] = on ? base + f->off_s[p] : nullptr;
  }
  m.x = x; m.y = y; m.z = z;
  m.out = f->d.out; m.in = f->d.in; m.k = f->d.k; m.n_paths = f->d.n_paths;
  m.rank = f->d.rank; m.scale_fmt = f->d.scale_fmt; m.row_stride = f->row_stride;
  m.groups = f->groups; m.ldx = ldx; m.ldy = ldy; m.batch = batch;
  m.terms = f->d.n_paths * f->d.rank;
  return m;
}

// Rows per wavefront for a single matrix: enough tiles to cover the chip
// about twice, at most kRowsMax.
uint32_t rows_per_wave_single(uint32_t out) {
  const uint32_t target_tiles = 512;
  uint32_t rw = (out + target_tiles * kWavesPerBlock - 1) / (target_tiles * kWavesPerBlock);
  if (rw < 1) rw = 1;
  if (rw > 32) rw = 32;
  return rw;
}

constexpr uint32_t kGroupedRW = 16;

int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? WAL_OK : WAL_ERR_DEVICE;
}

uint64_t up64(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

}  // namespace

extern "C" {

int wal_gemv(const wal_info* info, const void* W_dev, const void* x_dev, int x_dtype, float* y_dev,
             void* ws_dev, size_t ws_bytes, void* stream) {
  int st = check_info(info);
  if (st) return st;
  if (!W_dev || !x_dev || !y_dev) return WAL_ERR_ARG;
  if (x_dtype != WAL_X_F32 && x_dtype != WAL_X_BF16) return WAL_ERR_ARG;
  if (!aligned(W_dev, 256) || !aligned(x_dev, 16) || !aligned(y_dev, 4)) return WAL_ERR_ALIGN;
  size_t need = 0;
  if ((st = wal_workspace_size(info, 1, &need))) return st;
  if (need && (!ws_dev || ws_bytes < need)) return ws_dev ? WAL_ERR_BUFFER : WAL_ERR_ARG;
  if (need && !aligned(ws_dev, 16)) return WAL_ERR_ALIGN;
  if (overlap(x_dev, (size_t)info->d.in * xelem(x_dtype), y_dev, (size_t)info->d.out * 4)) return WAL_ERR_ARG;
  if (info->d.trit_fmt != WAL_TRIT_2BIT) return WAL_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  MatDev d = make_dev(info, W_dev, x_dev, y_dev, static_cast<float*>(ws_dev), info->d.in, info->d.out, 1);
  if (d.terms) {
    const uint32_t g = (d.terms + kWavesPerBlock - 1) / kWavesPerBlock;
    if (x_dtype == WAL_X_BF16) hipLaunchKernelGGL(k_z_single<WAL_X_BF16>, dim3(g), dim3(kBlockThreads), 0, s, d);
    else hipLaunchKernelGGL(k_z_single<WAL_X_F32>, dim3(g), dim3(kBlockThreads), 0, s, d);
    if ((st = launch_status())) return st;
  }
  const uint32_t rw = rows_per_wave_single(d.out);
  const uint32_t grid = (d.out + kWavesPerBlock * rw - 1) / (kWavesPerBlock * rw);
  if (x_dtype == WAL_X_BF16) hipLaunchKernelGGL(k_gemv2_single<WAL_X_BF16>, dim3(grid), dim3(kBlockThreads), 0, s, d, rw);
  else hipLaunchKernelGGL(k_gemv2_single<WAL_X_F32>, dim3(grid), dim3(kBlockThreads), 0, s, d, rw);
  return launch_status();
}

int wal_gemm_small(const wal_info* info, const void* W_dev, const void* X_dev, int x_dtype, uint32_t batch,
                   uint32_t ldx, float* Y_dev, uint32_t ldy, int mode, void* ws_dev, size_t ws_bytes,
                   void* stream) {
  int st = check_info(info);
  if (st) return st;
  if (batch == 0 || batch > WAL_MAX_BATCH) return WAL_ERR_ARG;
  if (mode < WAL_GEMM_AUTO || mode > WAL_GEMM_MFMA) return WAL_ERR_ARG;
  if (batch == 1 && mode != WAL_GEMM_MFMA)
    return wal_gemv(info, W_dev, X_dev, x_dtype, Y_dev, ws_dev, ws_bytes, stream);
  (void)ldx; (void)ldy;
  return WAL_ERR_UNSUPPORTED;
}

int wal_grouped_plan_size(uint32_t n, const wal_info* infos, size_t* plan_bytes, size_t* ws_bytes) {
  if (!n || !infos || !plan_bytes || !ws_bytes) return WAL_ERR_ARG;
  uint64_t tiles = 0, jobs = 0, ws = 0;
  for (uint32_t i = 0; i < n; ++i) {
    int st = check_info(&infos[i]);
    if (st) return st;
    const uint32_t rows_per_tile = kWavesPerBlock * kGroupedRW;
    tiles += (infos[i].d.out + rows_per_tile - 1) / rows_per_tile;
    jobs += infos[i].d.n_paths * infos[i].d.rank;
    ws += up64(4ull * infos[i].d.n_paths * infos[i].d.rank, 16);
  }
  uint64_t b = up64(sizeof(PlanHeader), 64);
  b += up64((uint64_t)n * sizeof(MatDev), 64);
  b += up64(tiles * 8, 64);
  b += up64(jobs * 4, 64);
  *plan_bytes = (size_t)b;
  *ws_bytes = (size_t)up64(ws, 256);
  return WAL_OK;
}

int wal_grouped_plan(uint32_t n, const wal_info* infos, const void* const* W_dev, const void* const* x_dev,
                     int x_dtype, float* const* y_dev, void* ws_dev, size_t ws_bytes, void* plan_host,
                     size_t plan_bytes, wal_grouped_info* ginfo) {
  size_t need_plan = 0, need_ws = 0;
  int st = wal_grouped_plan_size(n, infos, &need_plan, &need_ws);
  if (st) return st;
  if (!W_dev || !x_dev || !y_dev || !plan_host || !ginfo) return WAL_ERR_ARG;
  if (x_dtype != WAL_X_F32 && x_dtype != WAL_X_BF16) return WAL_ERR_ARG;
  if (plan_bytes < need_plan) return WAL_ERR_BUFFER;
  if (need_ws && (!ws_dev || ws_bytes < need_ws)) return ws_dev ? WAL_ERR_BUFFER : WAL_ERR_ARG;
  if (need_ws && !aligned(ws_dev, 16)) return WAL_ERR_ALIGN;
  const uint32_t tf = infos[0].d.trit_fmt;
  for (uint32_t i = 0; i < n; ++i) {
    if (!W_dev[i] || !x_dev[i] || !y_dev[i]) return WAL_ERR_ARG;
    if (!aligned(W_dev[i], 256) || !aligned(x_dev[i], 16) || !aligned(y_dev[i], 4)) return WAL_ERR_ALIGN;
    if (infos[i].d.trit_fmt != tf) return WAL_ERR_ARG;
    if (overlap(x_dev[i], (size_t)infos[i].d.in * xelem(x_dtype), y_dev[i], (size_t)infos[i].d.out * 4))
      return WAL_ERR_ARG;
  }
  if (tf != WAL_TRIT_2BIT) return WAL_ERR_UNSUPPORTED;
  uint8_t* base = static_cast<uint8_t*>(plan_host);
  std::memset(base, 0, need_plan);
  PlanHeader* h = reinterpret_cast<PlanHeader*>(base);
  h->magic = kPlanMagic;
  h->n = n;
  h->rows_per_wave = kGroupedRW;
  h->x_dtype = (uint32_t)x_dtype;
  h->trit_fmt = tf;
  h->off_descs = up64(sizeof(PlanHeader), 64);
  MatDev* descs = reinterpret_cast<MatDev*>(base + h->off_descs);
  uint64_t zoff = 0, tiles = 0, jobs = 0;
  const uint32_t rows_per_tile = kWavesPerBlock * kGroupedRW;
  for (uint32_t i = 0; i < n; ++i) {
    float* z = static_cast<float*>(ws_dev) + zoff / 4;
    descs[i] = make_dev(&infos[i], W_dev[i], x_dev[i], y_dev[i], infos[i].d.n_paths ? z : nullptr,
                        infos[i].d.in, infos[i].d.out, 1);
    zoff += up64(4ull * infos[i].d.n_paths * infos[i].d.rank, 16);
    tiles += (infos[i].d.out + rows_per_tile - 1) / rows_per_tile;
    jobs += infos[i].d.n_paths * infos[i].d.rank;
  }
  h->n_tiles = (uint32_t)tiles;
  h->n_zjobs = (uint32_t)jobs;
  h->off_tiles = h->off_descs + up64((uint64_t)n * sizeof(MatDev), 64);
  h->off_zjobs = h->off_tiles + up64(tiles * 8, 64);
  h->bytes = need_plan;
  uint32_t* tl = reinterpret_cast<uint32_t*>(base + h->off_tiles);
  uint32_t* jb = reinterpret_cast<uint32_t*>(base + h->off_zjobs);
  uint64_t t = 0, j = 0;
  for (uint32_t i = 0; i < n; ++i) {
    for (uint32_t r0 = 0; r0 < infos[i].d.out; r0 += rows_per_tile, ++t) { tl[2 * t] = i; tl[2 * t + 1] = r0; }
    for (uint32_t q = 0; q < infos[i].d.n_paths * infos[i].d.rank; ++q, ++j) jb[j] = (i << 8) | q;
  }
  std::memset(ginfo, 0, sizeof(*ginfo));
  ginfo->n = n;
  ginfo->n_tiles = h->n_tiles;
  ginfo->n_zjobs = h->n_zjobs;
  ginfo->rows_per_wave = kGroupedRW;
  ginfo->x_dtype = (uint32_t)x_dtype;
  ginfo->trit_fmt = tf;
  ginfo->grid = h->n_tiles < 1024 ? h->n_tiles : 1024;
  ginfo->plan_bytes = need_plan;
  uint64_t alg = 0;
  for (uint32_t i = 0; i < n; ++i) alg += infos[i].algorithmic_bytes;
  ginfo->algorithmic_bytes = alg;
  return WAL_OK;
}

int wal_gemv_grouped(const wal_grouped_info* g, const void* plan_dev, void* stream) {
  if (!g || !plan_dev) return WAL_ERR_ARG;
  if (!aligned(plan_dev, 16)) return WAL_ERR_ALIGN;
  if (g->x_dtype > WAL_X_BF16 || g->trit_fmt != WAL_TRIT_2BIT || !g->n || !g->grid) return WAL_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* base = static_cast<const uint8_t*>(plan_dev);
  const uint64_t off_descs = up64(sizeof(PlanHeader), 64);
  const uint64_t off_tiles = off_descs + up64((uint64_t)g->n * sizeof(MatDev), 64);
  const uint64_t off_jobs = off_tiles + up64((uint64_t)g->n_tiles * 8, 64);
  const MatDev* descs = reinterpret_cast<const MatDev*>(base + off_descs);
  const uint2* tiles = reinterpret_cast<const uint2*>(base + off_tiles);
  const uint32_t* jobs = reinterpret_cast<const uint32_t*>(base + off_jobs);
  int st;
  if (g->n_zjobs) {
    const uint32_t grid = (g->n_zjobs + kWavesPerBlock - 1) / kWavesPerBlock;
    if (g->x_dtype == WAL_X_BF16)
      hipLaunchKernelGGL(k_z_grouped<WAL_X_BF16>, dim3(grid), dim3(kBlockThreads), 0, s, descs, jobs, g->n_zjobs);
    else
      hipLaunchKernelGGL(k_z_grouped<WAL_X_F32>, dim3(grid), dim3(kBlockThreads), 0, s, descs, jobs, g->n_zjobs);
    if ((st = launch_status())) return st;
  }
  if (g->x_dtype == WAL_X_BF16)
    hipLaunchKernelGGL(k_gemv2_grouped<WAL_X_BF16>, dim3(g->grid), dim3(kBlockThreads), 0, s, descs, tiles,
                       g->n_tiles, g->rows_per_wave);
  else
    hipLaunchKernelGGL(k_gemv2_grouped<WAL_X_F32>, dim3(g->grid), dim3(kBlockThreads), 0, s, descs, tiles,
                       g->n_tiles, g->rows_per_wave);
  return launch_status();
}

}  // extern "C"
