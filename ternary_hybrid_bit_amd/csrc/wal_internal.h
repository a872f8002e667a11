// Internal declarations shared by the host code and the HIP kernels of libwal.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/wal.h"

namespace wal {

// Device-side descriptor of one matrix: plane pointers, activation, output
// and workspace slot.  Built on the host, read by the kernels (by value for a
// single product, from the plan blob for grouped products).
struct MatDev {
  const uint8_t* codes;
  const uint8_t* sites;
  const uint8_t* alpha;
  const uint8_t* beta;
  const uint8_t* V[WAL_MAX_PATHS];
  const uint8_t* U[WAL_MAX_PATHS];
  const uint8_t* s[WAL_MAX_PATHS];
  const void* x;       // [batch][ldx] activations
  float* y;            // [batch][ldy] outputs
  float* z;            // [batch][n_paths * rank] workspace: diag(s_p) V_p^T x
  uint32_t out, in, k, n_paths, rank, scale_fmt, row_stride, groups;
  uint32_t ldx, ldy, batch, terms;  // terms = n_paths * rank
};

// Plan blob written by wal_grouped_plan (host) and read by the kernels.
struct PlanHeader {
  uint32_t magic, n, n_tiles, n_zjobs, rows_per_wave, x_dtype, trit_fmt, reserved;
  uint64_t off_descs, off_tiles, off_zjobs, bytes;
};
constexpr uint32_t kPlanMagic = 0x4E4C5057u;  // "WPLN"

// Columns one wavefront covers per pass: 64 lanes x 16 bytes of codes.
constexpr uint32_t kPass2bit = 4096;   // 2-bit: 64 trits per lane
constexpr uint32_t kPassBase3 = 5120;  // base-3: 80 trits per lane
constexpr uint32_t kWavesPerBlock = 8;
constexpr uint32_t kBlockThreads = 64 * kWavesPerBlock;

// Host helpers implemented in wal_host.cpp / wal_gpu.hip.
int check_info(const wal_info* info);

}  // namespace wal
