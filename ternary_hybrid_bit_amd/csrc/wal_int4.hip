// INT4/g128 and INT5/g128 GEMV for gfx950 (the WAL-Ternary-8B cards' LM
// head, INT4/g128, and the WAL-Ternary-27B-RC1 card's packed INT5 head):
//     y[v] = sum_g s[v][g] sum_{j in g} q[v][j] x[j]
// with q signed codes (INT4: two per byte, element 2i low; INT5: an LSB-first
// 5-bit stream per row) and one fp16 scale per 128 columns (layouts in
// include/wal.h); and the embedding-row lookup of INT3 and INT4 tables.
//
// A wavefront takes kI4Rows rows at a time over one 4096-column pass, 64
// columns per lane, read so that every load instruction covers contiguous
// bytes across the lanes: INT4 lane l takes the 32-column pieces at 32 l and
// 2048 + 32 l (16 code bytes and one scale each); INT5 lane l takes columns
// 64 l .. 64 l + 63 (40 code bytes, half a scale group), whose codes the
// wavefront loads as contiguous 16-byte chunks and passes through LDS.
// Codes are flipped to offset binary and spread into bf16 pairs
// 0x4300 | (q + 2^(b-1)) = 128 + 2^(b-1) + q, which feed v_dot2_f32_bf16
// against x pairs arranged to match (INT4: columns k and k + 4 of a dword,
// INT5: columns 2 m and 2 m + 1); the sum of the offset times x over the
// lane's columns, formed by the same v_dot2 sequence, comes off once per row,
// so it cancels exactly.  x and that sum stay in registers for widths up to
// one pass (plus a 1024-column tail spread over the wavefront); the next
// batch's codes and scales are loaded while one batch is reduced, and the
// rows' lane sums meet in one transposed butterfly.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "wal_device.h"
#include "wal_internal.h"

namespace {

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

constexpr int kI4Rows = 4;        // rows per batch of a wavefront (a power of two, at most 32)
static_assert(kI4Rows >= 2 && kI4Rows <= 32 && (kI4Rows & (kI4Rows - 1)) == 0, "rows per batch");
constexpr uint32_t kI4Pass = 4096;

template <int BITS, int NR> struct QBatch;
// INT4: the lane's 64 columns are two 32-column pieces (16 code bytes and
// one scale each): columns c and c + gap, gap = 2048 in a pass, so that each
// load instruction reads 1 KB contiguous over the wavefront.
template <int NR> struct QBatch<4, NR> {
  u32x4_t c[NR][2];   // 16 code bytes per piece
  uint32_t s[NR][2];  // scale bits per piece
};
// INT5 codes travel as 16-byte chunks contiguous across the wavefront's
// lanes (chunk j = lane + 64 k of the batch's NR row pieces of 2560 bytes)
// and reach their lanes through LDS (stage5).
template <int NR> constexpr int kI5Chunks = (NR * 160 + 63) / 64;
template <int NR> struct QBatch<5, NR> {
  u32x4_t c[kI5Chunks<NR>];
  uint32_t s[NR];
};

// x of the lane for one pass, and base = the sum of (offset) x over the
// lane's columns formed by the same v_dot2 sequence as a row's sum, so that
// it cancels exactly: all-zero codes give exactly 0 and a basis vector
// x = e_j gives s q exactly (columns past `in` read as zero).
//   INT4: p[d][k] = (x[c + 8 d + k], x[c + 8 d + k + 4]) for code dword d < 4
//         of the first piece (c its first column; d >= 4: the second piece)
//         and nibble pair k; offset 136, one base per piece.
//   INT5: p[m] = (x[64 l + 2 m], x[64 l + 2 m + 1]); offset 144.
template <int BITS> struct QX;
template <> struct QX<4> {
  uint32_t p[8][4];
  float base[2];
};
template <> struct QX<5> {
  uint32_t p[32];
  float base;
};

constexpr uint32_t kBf16Pair136 = 0x43084308u;   // bf16 (136, 136)
constexpr uint32_t kBf16Pair144 = 0x43104310u;   // bf16 (144, 144)

__device__ __forceinline__ void load_x_pairs(__amdgpu_buffer_rsrc_t rx, uint32_t col, uint32_t (&w)[32]) {
  // bf16 pairs (x[2m], x[2m + 1]) of the lane's 64 columns
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rx, 2 * col + 16 * k, 0, 0);
    w[4 * k] = v[0]; w[4 * k + 1] = v[1]; w[4 * k + 2] = v[2]; w[4 * k + 3] = v[3];
  }
}

// INT4: pieces at columns col and col + gap
__device__ __forceinline__ void load_x(__amdgpu_buffer_rsrc_t rx, uint32_t col, uint32_t gap, QX<4>& X) {
  uint32_t w[32];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rx, 2 * (col + (k >= 4 ? gap : 0)) + 16 * (k & 3), 0, 0);
    w[4 * k] = v[0]; w[4 * k + 1] = v[1]; w[4 * k + 2] = v[2]; w[4 * k + 3] = v[3];
  }
  float base[2] = {0.f, 0.f};
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    // columns 8 d .. 8 d + 7 are bf16 pairs w[4 d] .. w[4 d + 3]
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = w[4 * d + (k >> 1)], hi = w[4 * d + 2 + (k >> 1)];
      // column 8 d + k from lo (half k & 1), column 8 d + k + 4 from hi
      X.p[d][k] = __builtin_amdgcn_perm(hi, lo, (k & 1) ? 0x07060302u : 0x05040100u);
      base[d >> 2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kBf16Pair136),
                                                     __builtin_bit_cast(bf16x2_t, X.p[d][k]), base[d >> 2], false);
    }
  }
  X.base[0] = base[0];
  X.base[1] = base[1];
}

__device__ __forceinline__ void load_x(__amdgpu_buffer_rsrc_t rx, uint32_t col, QX<5>& X) {
  load_x_pairs(rx, col, X.p);
  float base = 0.f;
#pragma unroll
  for (int m = 0; m < 32; ++m)
    base = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kBf16Pair144),
                                           __builtin_bit_cast(bf16x2_t, X.p[m]), base, false);
  X.base = base;
}

// Row r of a batch at matrix row `row`: INT4 the pieces at col and
// col + gap (codes and scales), INT5 the scale of the 64 columns from col
// (its codes: load5).  A column >= in (past a partial last pass, or an idle
// tail lane) sets bit 31 of the offsets (the matrix is under 2^31 bytes), so
// the loads read out of range, zeros, which meet x = 0 there.  (A select
// between two offsets here becomes a branch around every load.)
template <int BITS, int NR>
__device__ __forceinline__ void load_row(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, QBatch<BITS, NR>& B,
                                         int r, uint32_t row, uint32_t col, uint32_t in, uint32_t gap = 0) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t c = col + (h ? gap : 0), oob = (uint32_t)(c >= in) << 31;
      // read once: streaming policy
      B.c[r][h] = __builtin_amdgcn_raw_buffer_load_b128(rc, (row * (in / 2) + c / 2) | oob, 0, kStream);
      B.s[r][h] = __builtin_amdgcn_raw_buffer_load_b16(rs, (2 * (row * (in / 128) + c / 128)) | oob, 0, 0);
    }
  } else {
    const uint32_t oob = (uint32_t)(col >= in) << 31;
    B.s[r] = __builtin_amdgcn_raw_buffer_load_b16(rs, (2 * (row * (in / 128) + col / 128)) | oob, 0, 0);
  }
}

// INT4: kI4Rows rows from row0 at one pass's pieces (col, col + kI4Gap),
// and with a tail (NR = kI4Rows + 1) one more row's 64 columns: row
// row0 + trow at tcol (pieces tcol, tcol + 32).
constexpr uint32_t kI4Gap = 2048;
template <int NR>
__device__ __forceinline__ QBatch<4, NR> load_rows(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                                   uint32_t row0, uint32_t V, uint32_t in, uint32_t col,
                                                   uint32_t trow, uint32_t tcol) {
  QBatch<4, NR> B;
#pragma unroll
  for (int r = 0; r < kI4Rows; ++r) load_row(rc, rs, B, r, min(row0 + r, V - 1), col, in, kI4Gap);
  if constexpr (NR > kI4Rows) load_row(rc, rs, B, kI4Rows, min(row0 + trow, V - 1), tcol, in, 32u);
  return B;
}

// Row r's share of the lane: per piece s * (sum of (136 + q) x - sum of 136 x)
template <int NR>
__device__ __forceinline__ float dot_row(const QBatch<4, NR>& B, int r, const QX<4>& X) {
  float a[2] = {0.f, 0.f};   // one sum per piece
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const uint32_t w = B.c[r][d >> 2][d & 3] ^ 0x88888888u;   // offset binary: q + 8
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t pr = ((w >> (4 * k)) & 0x000F000Fu) | 0x43004300u;   // (136 + q_k, 136 + q_{k+4})
      a[d >> 2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pr),
                                                  __builtin_bit_cast(bf16x2_t, X.p[d][k]), a[d >> 2], false);
    }
  }
  return (float)__builtin_bit_cast(_Float16, (uint16_t)B.s[r][0]) * (a[0] - X.base[0]) +
         (float)__builtin_bit_cast(_Float16, (uint16_t)B.s[r][1]) * (a[1] - X.base[1]);
}

// INT5: s * (sum of (144 + q) x - sum of 144 x).  Pair m is the 10-bit field
// at window bit 10 m (codes of columns 2 m, 2 m + 1, two's complement): a
// shift-or spreads it to bits 0..4 and 16..20, and one three-input bitwise op
// keeps those bits, flips each code's sign bit (q + 16, offset binary) and
// sets the exponent, giving the bf16 pair 0x4300 | (q + 16) = 144 + q.
__device__ __forceinline__ float dot5(const uint32_t (&w)[10], uint32_t sbits, const QX<5>& X) {
  float a = 0.f;
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const int d = (10 * m) >> 5, o = (10 * m) & 31;
    const uint32_t f = (o <= 22 ? (w[d] >> o) : __builtin_amdgcn_alignbit(w[d < 9 ? d + 1 : 9], w[d], o)) & 0x3FFu;
    // (S0 & S1) ^ S2: truth table 0x6A over (S0, S1, S2) = bit index 4 S0 + 2 S1 + S2
    const uint32_t pr = __builtin_amdgcn_bitop3_b32((f << 11) | f, 0x001F001Fu, 0x43104310u, 0x6A);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pr), __builtin_bit_cast(bf16x2_t, X.p[m]), a,
                                       false);
  }
  return (float)__builtin_bit_cast(_Float16, (uint16_t)sbits) * (a - X.base);
}

// Per-lane offsets of the INT5 chunks of one pass (added to the batch's
// first row times the row bytes).  Piece r < kI4Rows is row r's 2560 bytes
// from pass byte cb0 (chunks at or past the pass's `pbytes` read zeros);
// piece kI4Rows (the tail) holds the kI4Rows rows' tails of T lane pieces
// (40 T bytes each, T even) one after another, so that lane l finds piece
// l % T of row l / T at byte 40 l, as it finds its columns of a full row.
// Unused chunks set only bit 31: row base + 2^31 stays below 2^32 and past
// the codes, so they read zeros.
template <int NR>
struct Plan5 {
  uint32_t off[kI5Chunks<NR>];
};

template <int NR>
__device__ __forceinline__ Plan5<NR> plan5(uint32_t lane, uint32_t rowbytes, uint32_t cb0, uint32_t pbytes,
                                           uint32_t T) {
  Plan5<NR> P;
#pragma unroll
  for (int k = 0; k < kI5Chunks<NR>; ++k) {
    const uint32_t j = lane + 64 * k, piece = j / 160, c = j - 160 * piece;
    uint32_t off = 0x80000000u;
    if (piece < kI4Rows) {
      if (16 * c < pbytes) off = piece * rowbytes + cb0 + 16 * c;
    } else if (piece == kI4Rows && c < 10 * T) {
      const uint32_t per = 5 * T / 2, r = c / per;
      off = r * rowbytes + kI4Pass * 5 / 8 + 16 * (c - r * per);
    }
    P.off[k] = off;
  }
  return P;
}

// Through the wavefront's LDS slice `sl` (NR * 160 chunks as 8-byte
// halves): chunks in, then piece r's 40 bytes of this lane out.  The lanes
// read what other lanes wrote: a wave-level hand-off before the writes (the
// previous batch's reads come first) and after them (every write lands
// before the reads).  Without it the compiler dropped or sank writes that
// the writing lane never reads back itself.
template <int NR>
__device__ __forceinline__ void stage5(u32x2_t* sl, const QBatch<5, NR>& B, uint32_t lane) {
  wave_lds_sync();   // the previous batch's reads come first
#pragma unroll
  for (int k = 0; k < kI5Chunks<NR>; ++k)
    if ((NR * 160) % 64 == 0 || k + 1 < kI5Chunks<NR> || lane + 64 * k < NR * 160) {
      const u32x4_t c = B.c[k];
      sl[2 * (lane + 64 * k)] = u32x2_t{c[0], c[1]};
      sl[2 * (lane + 64 * k) + 1] = u32x2_t{c[2], c[3]};
    }
  wave_lds_sync();   // every write lands before the reads
}

__device__ __forceinline__ void unstage5(const u32x2_t* sl, int r, uint32_t lane, uint32_t (&w)[10]) {
  const u32x2_t* p = sl + r * 320 + 5 * lane;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const u32x2_t v = p[i];
    w[2 * i] = v[0];
    w[2 * i + 1] = v[1];
  }
}

// Sum of acc[r] over the wavefront's 64 lanes by a transposed butterfly:
// each xor step from 32 down halves the rows a lane keeps (the lane with the
// step's bit set keeps the upper half), until each lane holds one row, then
// the last steps add that row over the lanes that share it.  The row of lane
// l is reduce_row(l); the lanes with l & (64 / kI4Rows - 1) == 0 hold sums.
__device__ __forceinline__ uint32_t reduce_row(uint32_t lane) {
  uint32_t row = 0;
#pragma unroll
  for (int m = 32, half = kI4Rows / 2; half >= 1; m >>= 1, half >>= 1)
    if (lane & m) row += half;
  return row;
}

__device__ __forceinline__ float reduce_rows(const float (&acc)[kI4Rows], uint32_t lane) {
  float v[kI4Rows];
#pragma unroll
  for (int r = 0; r < kI4Rows; ++r) v[r] = acc[r];
  int m = 32;
#pragma unroll
  for (int half = kI4Rows / 2; half >= 1; half >>= 1, m >>= 1) {
    const bool upper = lane & m;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float keep = upper ? v[i + half] : v[i], send = upper ? v[i] : v[i + half];
      v[i] = keep + __shfl_xor(send, m);
    }
  }
  float t = v[0];
#pragma unroll
  for (; m >= 1; m >>= 1) t += __shfl_xor(t, m);
  return t;
}

// A wavefront per batch of kI4Rows rows, grid-stride over the batches.
// Widths up to one pass keep x in registers with two batches in flight;
// widths up to one pass + 1024 columns (the 27B models' 5120) add a tail:
// the kI4Rows rows' remaining T = (in - 4096) / 64 lane pieces are spread
// over the wavefront, lane l taking piece l % T of row l / T, so that one
// extra load per lane covers all of them (every lane busy when T = 16);
// wider matrices take one pass after another.
enum { kPathOne = 0, kPathTail = 1, kPathMulti = 2 };

__host__ __device__ constexpr int qgemv_path(uint32_t in) {
  return in <= kI4Pass ? kPathOne : in <= kI4Pass + 1024 ? kPathTail : kPathMulti;
}

template <int PATH>
__device__ __forceinline__ void qgemv4(const uint8_t* __restrict__ W, uint32_t V, uint32_t in,
                                      const void* __restrict__ x, float* __restrict__ y) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = blockIdx.x * 4 + (threadIdx.x >> 6), nwaves = gridDim.x * 4;
  const uint32_t batches = (V + kI4Rows - 1) / kI4Rows;
  const uint32_t npass = (in + kI4Pass - 1) / kI4Pass;
  const uint32_t cbytes = V * (in / 2);
  const __amdgpu_buffer_rsrc_t rc = rsrc(W, cbytes);
  const __amdgpu_buffer_rsrc_t rs = rsrc(W + cbytes, V * (in / 128) * 2);
  const __amdgpu_buffer_rsrc_t rx = rsrc(x, 2 * in);
  uint32_t b = wave;
  if (b >= batches) return;
  QX<4> X;
  load_x(rx, 32 * lane, kI4Gap, X);
  if constexpr (PATH == kPathOne) {
    QBatch<4, kI4Rows> B0 = load_rows<kI4Rows>(rc, rs, b * kI4Rows, V, in, 32 * lane, 0, 0);
    for (;;) {
      const uint32_t bn = b + nwaves;
      const QBatch<4, kI4Rows> B1 =
          load_rows<kI4Rows>(rc, rs, min(bn, batches - 1) * kI4Rows, V, in, 32 * lane, 0, 0);
      float acc[kI4Rows];
#pragma unroll
      for (int r = 0; r < kI4Rows; ++r) acc[r] = dot_row(B0, r, X);
      const float v = reduce_rows(acc, lane);
      const uint32_t row = b * kI4Rows + reduce_row(lane);
      if ((lane & (64 / kI4Rows - 1)) == 0 && row < V) y[row] = v;
      if (bn >= batches) break;
      b = bn;
      B0 = B1;
    }
  } else if constexpr (PATH == kPathTail) {
    const uint32_t T = (in - kI4Pass) / 64, trow = lane / T;
    const uint32_t tcol = trow < kI4Rows ? kI4Pass + 64 * (lane % T) : in;   // idle lanes read zeros
    QX<4> XT;
    load_x(rx, tcol, 32u, XT);
    constexpr int NR = kI4Rows + 1;
    QBatch<4, NR> B0 = load_rows<NR>(rc, rs, b * kI4Rows, V, in, 32 * lane, trow, tcol);
    for (;;) {
      const uint32_t bn = b + nwaves;
      const QBatch<4, NR> B1 =
          load_rows<NR>(rc, rs, min(bn, batches - 1) * kI4Rows, V, in, 32 * lane, trow, tcol);
      const float t = dot_row(B0, kI4Rows, XT);
      float acc[kI4Rows];
#pragma unroll
      for (int r = 0; r < kI4Rows; ++r) acc[r] = dot_row(B0, r, X) + (trow == (uint32_t)r ? t : 0.f);
      const float v = reduce_rows(acc, lane);
      const uint32_t row = b * kI4Rows + reduce_row(lane);
      if ((lane & (64 / kI4Rows - 1)) == 0 && row < V) y[row] = v;
      if (bn >= batches) break;
      b = bn;
      B0 = B1;
    }
  } else {
    for (; b < batches; b += nwaves) {
      float acc[kI4Rows] = {};
      for (uint32_t p = 0; p < npass; ++p) {
        // X holds pass 0 only before the wavefront's first batch
        if (p || b != wave) load_x(rx, p * kI4Pass + 32 * lane, kI4Gap, X);
        const QBatch<4, kI4Rows> B =
            load_rows<kI4Rows>(rc, rs, b * kI4Rows, V, in, p * kI4Pass + 32 * lane, 0, 0);
#pragma unroll
        for (int r = 0; r < kI4Rows; ++r) acc[r] += dot_row(B, r, X);
      }
      const float v = reduce_rows(acc, lane);
      const uint32_t row = b * kI4Rows + reduce_row(lane);
      if ((lane & (64 / kI4Rows - 1)) == 0 && row < V) y[row] = v;
    }
  }
}

// INT5: the same split as qgemv4, with the codes of a batch loaded as
// contiguous 16-byte chunks and handed to their lanes through the
// wavefront's LDS slice `sl` (NR * 320 eight-byte halves).
template <int NR>
__device__ __forceinline__ QBatch<5, NR> load5(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                               const Plan5<NR>& P, uint32_t row0, uint32_t V, uint32_t in,
                                               uint32_t rowbytes, uint32_t col, uint32_t trow, uint32_t tcol) {
  QBatch<5, NR> B;
  const uint32_t base = row0 * rowbytes;   // rows past V read zeros (past the codes)
#pragma unroll
  for (int k = 0; k < kI5Chunks<NR>; ++k)
    B.c[k] = __builtin_amdgcn_raw_buffer_load_b128(rc, P.off[k] + base, 0, kStream);
#pragma unroll
  for (int r = 0; r < kI4Rows; ++r) load_row(rc, rs, B, r, min(row0 + r, V - 1), col, in);
  if constexpr (NR > kI4Rows) load_row(rc, rs, B, kI4Rows, min(row0 + trow, V - 1), tcol, in);
  return B;
}

template <int PATH>
__device__ __forceinline__ void qgemv5(const uint8_t* __restrict__ W, uint32_t V, uint32_t in,
                                       const void* __restrict__ x, float* __restrict__ y, u32x2_t* sl) {
  constexpr int NR = PATH == kPathTail ? kI4Rows + 1 : kI4Rows;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = blockIdx.x * 4 + (threadIdx.x >> 6), nwaves = gridDim.x * 4;
  const uint32_t batches = (V + kI4Rows - 1) / kI4Rows;
  const uint32_t npass = (in + kI4Pass - 1) / kI4Pass;
  const uint32_t rowbytes = in * 5 / 8, cbytes = V * rowbytes;
  const __amdgpu_buffer_rsrc_t rc = rsrc(W, cbytes);
  const __amdgpu_buffer_rsrc_t rs = rsrc(W + cbytes, V * (in / 128) * 2);
  const __amdgpu_buffer_rsrc_t rx = rsrc(x, 2 * in);
  uint32_t b = wave;
  if (b >= batches) return;
  QX<5> X;
  load_x(rx, 64 * lane, X);
  uint32_t w[10];
  if constexpr (PATH == kPathOne) {
    const Plan5<NR> P = plan5<NR>(lane, rowbytes, 0, rowbytes, 0);
    QBatch<5, NR> B0 = load5<NR>(rc, rs, P, b * kI4Rows, V, in, rowbytes, 64 * lane, 0, 0);
    for (;;) {
      const uint32_t bn = b + nwaves;
      const QBatch<5, NR> B1 = load5<NR>(rc, rs, P, min(bn, batches - 1) * kI4Rows, V, in, rowbytes, 64 * lane, 0, 0);
      stage5(sl, B0, lane);
      float acc[kI4Rows];
#pragma unroll
      for (int r = 0; r < kI4Rows; ++r) {
        unstage5(sl, r, lane, w);
        acc[r] = dot5(w, B0.s[r], X);
      }
      const float v = reduce_rows(acc, lane);
      const uint32_t row = b * kI4Rows + reduce_row(lane);
      if ((lane & (64 / kI4Rows - 1)) == 0 && row < V) y[row] = v;
      if (bn >= batches) break;
      b = bn;
      B0 = B1;
    }
  } else if constexpr (PATH == kPathTail) {
    const uint32_t T = (in - kI4Pass) / 64, trow = lane / T;
    const uint32_t tcol = trow < kI4Rows ? kI4Pass + 64 * (lane % T) : in;   // idle lanes read zeros
    QX<5> XT;
    load_x(rx, tcol, XT);
    const Plan5<NR> P = plan5<NR>(lane, rowbytes, 0, kI4Pass * 5 / 8, T);
    QBatch<5, NR> B0 = load5<NR>(rc, rs, P, b * kI4Rows, V, in, rowbytes, 64 * lane, trow, tcol);
    for (;;) {
      const uint32_t bn = b + nwaves;
      const QBatch<5, NR> B1 =
          load5<NR>(rc, rs, P, min(bn, batches - 1) * kI4Rows, V, in, rowbytes, 64 * lane, trow, tcol);
      stage5(sl, B0, lane);
      unstage5(sl, kI4Rows, lane, w);
      const float t = dot5(w, B0.s[kI4Rows], XT);
      float acc[kI4Rows];
#pragma unroll
      for (int r = 0; r < kI4Rows; ++r) {
        unstage5(sl, r, lane, w);
        acc[r] = dot5(w, B0.s[r], X) + (trow == (uint32_t)r ? t : 0.f);
      }
      const float v = reduce_rows(acc, lane);
      const uint32_t row = b * kI4Rows + reduce_row(lane);
      if ((lane & (64 / kI4Rows - 1)) == 0 && row < V) y[row] = v;
      if (bn >= batches) break;
      b = bn;
      B0 = B1;
    }
  } else {
    for (; b < batches; b += nwaves) {
      float acc[kI4Rows] = {};
      for (uint32_t p = 0; p < npass; ++p) {
        // X holds pass 0 only before the wavefront's first batch
        if (p || b != wave) load_x(rx, p * kI4Pass + 64 * lane, X);
        const uint32_t cb0 = p * (kI4Pass * 5 / 8);
        const Plan5<NR> P = plan5<NR>(lane, rowbytes, cb0, min(kI4Pass * 5 / 8, rowbytes - cb0), 0);
        const QBatch<5, NR> B = load5<NR>(rc, rs, P, b * kI4Rows, V, in, rowbytes, p * kI4Pass + 64 * lane, 0, 0);
        stage5(sl, B, lane);
#pragma unroll
        for (int r = 0; r < kI4Rows; ++r) {
          unstage5(sl, r, lane, w);
          acc[r] += dot5(w, B.s[r], X);
        }
      }
      const float v = reduce_rows(acc, lane);
      const uint32_t row = b * kI4Rows + reduce_row(lane);
      if ((lane & (64 / kI4Rows - 1)) == 0 && row < V) y[row] = v;
    }
  }
}

// one kernel per code width and path, so that each gets its own registers
template <int PATH>
__global__ __launch_bounds__(256) void k_int4_gemv(const uint8_t* __restrict__ W, uint32_t V, uint32_t in,
                                                   const void* __restrict__ x, float* __restrict__ y) {
  qgemv4<PATH>(W, V, in, x, y);
}

template <int PATH>
__global__ __launch_bounds__(256) void k_int5_gemv(const uint8_t* __restrict__ W, uint32_t V, uint32_t in,
                                                   const void* __restrict__ x, float* __restrict__ y) {
  // one LDS slice of the INT5 codes per wavefront
  __shared__ u32x2_t sm[4][(PATH == kPathTail ? kI4Rows + 1 : kI4Rows) * 320];
  qgemv5<PATH>(W, V, in, x, y, sm[threadIdx.x >> 6]);
}

}  // namespace

static int qgemv_launch(int bits, const void* W_dev, uint32_t V, uint32_t in, const void* x_dev, int x_dtype,
                        float* y_dev, void* stream) {
  if (!W_dev || !x_dev || !y_dev || !V || !in) return WAL_ERR_ARG;
  if (x_dtype != WAL_X_F32 && x_dtype != WAL_X_BF16) return WAL_ERR_ARG;
  if (in % 128) return WAL_ERR_SHAPE;
  if ((uint64_t)V * in * bits / 8 + (uint64_t)V * (in / 128) * 2 >= (1ull << 31)) return WAL_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(W_dev) & 255u) || (reinterpret_cast<uintptr_t>(x_dev) & 15u) ||
      (reinterpret_cast<uintptr_t>(y_dev) & 3u))
    return WAL_ERR_ALIGN;
  if (x_dtype != WAL_X_BF16) return WAL_ERR_UNSUPPORTED;
  const size_t wbytes = (size_t)V * in * bits / 8 + (size_t)V * (in / 128) * 2;
  if (overlaps(y_dev, (size_t)V * 4, W_dev, wbytes) || overlaps(y_dev, (size_t)V * 4, x_dev, (size_t)in * 2))
    return WAL_ERR_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return WAL_ERR_DEVICE;
  const uint32_t batches = (V + kI4Rows - 1) / kI4Rows;
  // Workgroups per CU, each wavefront looping over batches.  INT4: three
  // (on the 151936 x 4096 head about 1 % faster than two or four, 11 %
  // faster than one); INT5: two, all its registers allow at the 5120 width.
  const uint32_t blocks = std::min<uint32_t>((batches + 3) / 4, (uint32_t)cus * (bits == 4 ? 3 : 2));
  const uint8_t* W = static_cast<const uint8_t*>(W_dev);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 g(blocks), t(256);
  const int path = qgemv_path(in);
  if (bits == 4) {
    if (path == kPathOne) hipLaunchKernelGGL(k_int4_gemv<kPathOne>, g, t, 0, s, W, V, in, x_dev, y_dev);
    else if (path == kPathTail) hipLaunchKernelGGL(k_int4_gemv<kPathTail>, g, t, 0, s, W, V, in, x_dev, y_dev);
    else hipLaunchKernelGGL(k_int4_gemv<kPathMulti>, g, t, 0, s, W, V, in, x_dev, y_dev);
  } else {
    if (path == kPathOne) hipLaunchKernelGGL(k_int5_gemv<kPathOne>, g, t, 0, s, W, V, in, x_dev, y_dev);
    else if (path == kPathTail) hipLaunchKernelGGL(k_int5_gemv<kPathTail>, g, t, 0, s, W, V, in, x_dev, y_dev);
    else hipLaunchKernelGGL(k_int5_gemv<kPathMulti>, g, t, 0, s, W, V, in, x_dev, y_dev);
  }
  return hipGetLastError() == hipSuccess ? WAL_OK : WAL_ERR_DEVICE;
}

extern "C" int wal_int4_gemv(const void* W_dev, uint32_t V, uint32_t in, const void* x_dev, int x_dtype,
                             float* y_dev, void* stream) {
  return qgemv_launch(4, W_dev, V, in, x_dev, x_dtype, y_dev, stream);
}

extern "C" int wal_int5_gemv(const void* W_dev, uint32_t V, uint32_t in, const void* x_dev, int x_dtype,
                             float* y_dev, void* stream) {
  return qgemv_launch(5, W_dev, V, in, x_dev, x_dtype, y_dev, stream);
}

// ---------------------------------------------------------------------------
// Embedding rows: out[i][:] = row ids[i] of an INT3 (3-bit stream) or INT4
// matrix (layouts in include/wal.h), or of a mixed table (INT3 and INT4 rows
// and a row map).  Block (i, c) decodes columns 2048 c .. 2048 c + 2047 of
// token i, 16 consecutive values per thread: INT3 takes 6 bytes at
// 6 (j0 / 16) of the row's stream (three 16-bit loads), INT4 8 bytes; one
// fp16 scale per thread (16 values lie inside one group).
namespace {

// Values j0 .. j0 + 15 of row `row` of a [V][in] table (row < V); each
// s * q is exact in fp32.
template <int BITS>
__device__ __forceinline__ void decode16(const uint8_t* __restrict__ W, uint32_t V, uint32_t in, uint32_t row,
                                         uint32_t j0, float (&e)[16]) {
  const uint32_t G = in / 128;
  const uint32_t cbytes = V * (in * BITS / 8);
  const __amdgpu_buffer_rsrc_t rc = rsrc(W, cbytes);
  const __amdgpu_buffer_rsrc_t rs = rsrc(W + cbytes, V * G * 2);
  const uint32_t base = row * (in * BITS / 8) + j0 * BITS / 8;
  uint64_t v;
  if constexpr (BITS == 3) {
    v = (uint64_t)__builtin_amdgcn_raw_buffer_load_b16(rc, base, 0, 0) |
        ((uint64_t)__builtin_amdgcn_raw_buffer_load_b16(rc, base + 2, 0, 0) << 16) |
        ((uint64_t)__builtin_amdgcn_raw_buffer_load_b16(rc, base + 4, 0, 0) << 32);
  } else {
    const u32x2_t w = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rc, base, 0, 0));
    v = (uint64_t)w[0] | ((uint64_t)w[1] << 32);
  }
  const float sc =
      (float)__builtin_bit_cast(_Float16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, 2 * (row * G + j0 / 128), 0, 0));
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int code = (int)((v >> (BITS * k)) & ((1u << BITS) - 1u));
    const int q = code >= (1 << (BITS - 1)) ? code - (1 << BITS) : code;
    e[k] = sc * (float)q;   // exact: at most 3 or 4 bits times an fp16 scale
  }
}

template <int OT>
__device__ __forceinline__ void store16(void* __restrict__ out, uint32_t ldo, uint32_t i, uint32_t j0,
                                        const float (&e)[16]) {
  if constexpr (OT == WAL_X_F32) {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + (size_t)i * ldo + j0);
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = make_float4(e[4 * k], e[4 * k + 1], e[4 * k + 2], e[4 * k + 3]);
  } else {
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t a = __float_as_uint(e[2 * k]), b = __float_as_uint(e[2 * k + 1]);
      w[k] = ((a + 0x7FFFu + ((a >> 16) & 1u)) >> 16) | (((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16) << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + (size_t)i * ldo + j0);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

template <int BITS, int OT>
__global__ __launch_bounds__(128) void k_embed_rows(const uint8_t* __restrict__ W, uint32_t V, uint32_t in,
                                                    const int32_t* __restrict__ ids, void* __restrict__ out,
                                                    uint32_t ldo) {
  const uint32_t i = blockIdx.x, j0 = blockIdx.y * 2048 + 16 * threadIdx.x;
  if (j0 >= in) return;
  const uint32_t row = (uint32_t)ids[i];   // a negative index wraps past V
  float e[16] = {};                        // +0 everywhere in a row past the vocabulary
  if (row < V) decode16<BITS>(W, V, in, row, j0, e);
  store16<OT>(out, ldo, i, j0, e);
}

// Mixed table: vocabulary row v is row m = map[v] of the INT3 table (m >= 0)
// or row -1 - m of the INT4 table; the choice is uniform over a block.
template <int OT>
__global__ __launch_bounds__(128) void k_embed_mixed(const uint8_t* __restrict__ W3, uint32_t V3,
                                                     const uint8_t* __restrict__ W4, uint32_t V4, uint32_t in,
                                                     const int32_t* __restrict__ map, uint32_t V,
                                                     const int32_t* __restrict__ ids, void* __restrict__ out,
                                                     uint32_t ldo) {
  const uint32_t i = blockIdx.x, j0 = blockIdx.y * 2048 + 16 * threadIdx.x;
  if (j0 >= in) return;
  const uint32_t v = (uint32_t)ids[i];
  float e[16] = {};
  if (v < V) {
    const int32_t m = map[v];
    if (m >= 0) {
      if ((uint32_t)m < V3) decode16<3>(W3, V3, in, (uint32_t)m, j0, e);
    } else if ((uint32_t)(-1 - m) < V4) {
      decode16<4>(W4, V4, in, (uint32_t)(-1 - m), j0, e);
    }
  }
  store16<OT>(out, ldo, i, j0, e);
}

}  // namespace

static int embed_check(uint32_t in, uint32_t n, void* out_dev, int out_dtype, uint32_t ldo) {
  if (out_dtype != WAL_X_F32 && out_dtype != WAL_X_BF16) return WAL_ERR_ARG;
  if (in % 128) return WAL_ERR_SHAPE;
  if (ldo < in) return WAL_ERR_ARG;
  if (n > 0x7FFFFFFFu) return WAL_ERR_SHAPE;   // one workgroup row per token: the grid's x limit
  const size_t oe = out_dtype == WAL_X_BF16 ? 2 : 4;
  if ((reinterpret_cast<uintptr_t>(out_dev) & 15u) || (ldo * oe) % 16) return WAL_ERR_ALIGN;
  return WAL_OK;
}

extern "C" int wal_embed_rows(const void* W_dev, int bits, uint32_t V, uint32_t in, const int32_t* ids_dev, uint32_t n,
                              void* out_dev, int out_dtype, uint32_t ldo, void* stream) {
  if (!W_dev || !ids_dev || !out_dev || !V || !in || !n) return WAL_ERR_ARG;
  if (bits != 3 && bits != 4) return WAL_ERR_ARG;
  int st = embed_check(in, n, out_dev, out_dtype, ldo);
  if (st) return st;
  if ((uint64_t)V * in * bits / 8 + (uint64_t)V * (in / 128) * 2 >= (1ull << 32)) return WAL_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(W_dev) & 255u) || (reinterpret_cast<uintptr_t>(ids_dev) & 3u)) return WAL_ERR_ALIGN;
  const size_t obytes = ((size_t)(n - 1) * ldo + in) * (out_dtype == WAL_X_BF16 ? 2 : 4);
  if (overlaps(out_dev, obytes, W_dev, (size_t)V * in * bits / 8 + (size_t)V * (in / 128) * 2) ||
      overlaps(out_dev, obytes, ids_dev, (size_t)n * 4))
    return WAL_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(n, (in + 2047) / 2048), block(128);
  const uint8_t* W = static_cast<const uint8_t*>(W_dev);
  if (bits == 3 && out_dtype == WAL_X_F32) hipLaunchKernelGGL((k_embed_rows<3, WAL_X_F32>), grid, block, 0, s, W, V, in, ids_dev, out_dev, ldo);
  else if (bits == 3) hipLaunchKernelGGL((k_embed_rows<3, WAL_X_BF16>), grid, block, 0, s, W, V, in, ids_dev, out_dev, ldo);
  else if (out_dtype == WAL_X_F32) hipLaunchKernelGGL((k_embed_rows<4, WAL_X_F32>), grid, block, 0, s, W, V, in, ids_dev, out_dev, ldo);
  else hipLaunchKernelGGL((k_embed_rows<4, WAL_X_BF16>), grid, block, 0, s, W, V, in, ids_dev, out_dev, ldo);
  return hipGetLastError() == hipSuccess ? WAL_OK : WAL_ERR_DEVICE;
}

extern "C" int wal_embed_rows_mixed(const void* W3_dev, uint32_t V3, const void* W4_dev, uint32_t V4, uint32_t in,
                                    const int32_t* map_dev, uint32_t V, const int32_t* ids_dev, uint32_t n,
                                    void* out_dev, int out_dtype, uint32_t ldo, void* stream) {
  if (!W3_dev || !W4_dev || !map_dev || !ids_dev || !out_dev || !V3 || !V4 || !V || !in || !n) return WAL_ERR_ARG;
  int st = embed_check(in, n, out_dev, out_dtype, ldo);
  if (st) return st;
  if ((uint64_t)V3 * in * 3 / 8 + (uint64_t)V3 * (in / 128) * 2 >= (1ull << 32) ||
      (uint64_t)V4 * in / 2 + (uint64_t)V4 * (in / 128) * 2 >= (1ull << 32))
    return WAL_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(W3_dev) & 255u) || (reinterpret_cast<uintptr_t>(W4_dev) & 255u) ||
      (reinterpret_cast<uintptr_t>(map_dev) & 3u) || (reinterpret_cast<uintptr_t>(ids_dev) & 3u))
    return WAL_ERR_ALIGN;
  const size_t obytes = ((size_t)(n - 1) * ldo + in) * (out_dtype == WAL_X_BF16 ? 2 : 4);
  if (overlaps(out_dev, obytes, W3_dev, (size_t)V3 * in * 3 / 8 + (size_t)V3 * (in / 128) * 2) ||
      overlaps(out_dev, obytes, W4_dev, (size_t)V4 * in / 2 + (size_t)V4 * (in / 128) * 2) ||
      overlaps(out_dev, obytes, map_dev, (size_t)V * 4) || overlaps(out_dev, obytes, ids_dev, (size_t)n * 4))
    return WAL_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(n, (in + 2047) / 2048), block(128);
  const uint8_t* W3 = static_cast<const uint8_t*>(W3_dev);
  const uint8_t* W4 = static_cast<const uint8_t*>(W4_dev);
  if (out_dtype == WAL_X_F32)
    hipLaunchKernelGGL(k_embed_mixed<WAL_X_F32>, grid, block, 0, s, W3, V3, W4, V4, in, map_dev, V, ids_dev, out_dev, ldo);
  else
    hipLaunchKernelGGL(k_embed_mixed<WAL_X_BF16>, grid, block, 0, s, W3, V3, W4, V4, in, map_dev, V, ids_dev, out_dev, ldo);
  return hipGetLastError() == hipSuccess ? WAL_OK : WAL_ERR_DEVICE;
}
