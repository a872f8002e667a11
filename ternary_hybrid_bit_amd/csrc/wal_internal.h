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
  // Low-rank path 0's planes; path p's are pstride bytes further per path
  // (every path's V, U and s planes have the same sizes, and the blob layout
  // places them one path after another).
  const uint8_t* V;
  const uint8_t* U;
  const uint8_t* s;
  uint32_t pstride;
  const void* x;       // [batch][ldx] activations
  float* y;            // [batch][ldy] outputs
  float* z;            // workspace: diag(s_p) V_p^T x, zc partial sums over
                       // column chunks [zc][n_paths * rank] (streaming kernels)
  uint32_t out, in, k, n_paths, rank, scale_fmt, row_stride, groups;
  uint32_t ldx, ldy, batch, terms;  // terms = n_paths * rank
  uint32_t blob_bytes;              // bytes of the blob from codes on (< 2^32)
  uint32_t trit_fmt;
  uint32_t zc;                      // chunks of z to add
  // Grouped plans whose matrix runs its passes in separate workgroups:
  // per-pass partial sums P[pass][out] (workspace) and the word offset of
  // its arrival counters (one per 16 rows) from the plan's synchronisation
  // words.
  float* P;
  uint32_t cnt_off;
};

// Plan blob written by wal_grouped_plan (host) and read by the kernels:
//   header | MatDev[n] | zjobs u32[2 n_zjobs] (matrix, t0 << 16 | chunk) |
//   per (scale format, k) class:
//   blockseg u32[grid + 1] | segs Seg[...]
// Workgroup b of a class's streaming launch processes its
// segs[blockseg[b] .. blockseg[b + 1]).  The header is informative only
// (reserved = number of classes); launches take offsets from wal_grouped_info.
struct PlanHeader {
  uint32_t magic, n, grid, n_segs, n_zjobs, x_dtype, zjob_terms, reserved;
  uint64_t off_descs, off_zjobs, bytes;
};
// Rows [row0, row1) of matrix mat; pass1 = 0: every pass, else pass pass1 - 1
// only (row0 then a multiple of 16).
struct Seg {
  uint32_t mat, row0, row1, pass1;
};
constexpr uint32_t kPlanMagic = 0x324E4C50u;  // "PLN2"

// Streaming kernels: 4 wavefronts per workgroup.
constexpr uint32_t kWaves = 4;
constexpr uint32_t kThreads = 64 * kWaves;
// Columns one wavefront covers per pass: 64 lanes x 16 bytes of codes.
constexpr uint32_t kPass2bit = 4096;   // 2-bit: 64 trits per lane
constexpr uint32_t kPassBase3 = 5120;  // base-3: 80 trits per lane
// Rows of one segment of a streaming workgroup (its y values are staged in
// LDS): the plans split longer row ranges.  Sized so that three workgroups
// fit in a CU's LDS.
constexpr uint32_t kSegRows = 4096;
// Low-rank terms handled per workgroup of the V^T x pre-passes.
constexpr uint32_t kZTerms = 4;
// Low-rank terms of one job of a grouped plan: a plan with at most
// kZJobsFewMax jobs of kZTermsFew terms uses those (short jobs, done before
// the streaming workgroups need them), a larger plan jobs of kZTermsMany (few
// jobs, so that a fused launch spends few of its first workgroups on them).
constexpr uint32_t kZTermsFew = 4;
constexpr uint32_t kZTermsMany = 16;
constexpr uint32_t kZJobsFewMax = 64;
static_assert(kZTerms == kZTermsFew, "single products run the short jobs");
constexpr uint32_t kMaxTerms = WAL_MAX_PATHS * WAL_MAX_RANK;
static_assert(kMaxTerms <= kThreads, "one low-rank term per thread of a streaming workgroup");

// Synchronisation words of a launch that computes the low-rank pre-pass in
// its first workgroups (see wal_device.h, fused launches), u32 words in
// 128-byte lines at the start of the workspace.  Hundreds of workgroups that
// each touch one coherent word queue on it, so every word the whole launch
// touches is kept in kSyncReplicas copies, one line apart; workgroup b uses
// copy b % kSyncReplicas.
//   line 0:       word 0 the fallback count, word 1 set when a wait of the
//                 current call gave up (the later waiters then give up at
//                 once), words 16 + s the copies of launch slot s whose
//                 workgroups have all finished
//   lines 1..16:  the epoch, the number of calls made on the workspace
//                 (copy r: word 0 of line 1 + r); the low-rank partials of a
//                 call carry the tag 2 epoch + 1
//   lines 17..32: workgroups finished (copy r: word s of line 17 + r)
// Every call leaves them as it found them, except the epoch, which its last
// workgroup advances, and the fallback count: the workgroups whose bounded
// wait for the low-rank jobs gave up and which computed the terms themselves
// (their outputs are still exact).
constexpr uint32_t kSyncReplicas = 16;
constexpr uint32_t kSyncLine = 32;                                  // words per line
constexpr uint32_t kSyncFallback = 0;
constexpr uint32_t kSyncGaveUp = 1;
constexpr uint32_t kSyncSlotsDone = 16;                             // + slot
constexpr uint32_t kSyncEpoch = kSyncLine;                          // + kSyncLine r
constexpr uint32_t kSyncFinished = kSyncLine * (1 + kSyncReplicas);  // + kSyncLine r + slot
constexpr uint32_t kSyncBytes = 4352;                                // 33 lines, padded to 256 bytes
static_assert(4 * kSyncLine * (1 + 2 * kSyncReplicas) <= kSyncBytes && kSyncBytes % 256 == 0, "sync lines");
static_assert(WAL_MAX_CLASSES <= 16, "one finish word per launch slot in a line");
// Arrival counters of split products follow the synchronisation words, at a
// place and size that do not depend on the blob: a workspace that served
// one shape still has them zero for the next.
constexpr uint32_t kMaxRowBlocks = 4096;
constexpr uint32_t kWsZeroBytes = kSyncBytes + 4 * kMaxRowBlocks;

// What a fused launch does besides streaming.  Workgroups below nz compute
// low-rank job blockIdx.x, the others stream (block blockIdx.x - nz).
// Workgroups start in index order, so the jobs are under way before any
// streaming workgroup waits for them; the wait is bounded all the same, and
// a workgroup whose wait gives up computes the terms it needs itself.
// With zwait, consumers wait until every partial they read carries the
// call's tag; without, the partials are ready (a separate pre-pass).  The
// last workgroup to finish returns finished[slot] to zero, and after the
// call's last launch (last) advances the epoch.
struct Fuse {
  uint32_t* sync;       // the synchronisation words (null: no waits, no counts)
  uint32_t slot, nz, zwait, grid, last;
  uint32_t zterms;      // low-rank terms per job (kZTermsFew or kZTermsMany)
};

// Streaming kernels as host-side launch targets.
struct Seg;
// Grouped: (descriptors, block -> segment index, segments, low-rank jobs,
// launch context).
using GroupedFn = void (*)(const MatDev*, const uint32_t*, const Seg*, const uint32_t*, Fuse);
// Single-product streaming kernel: (descriptor, rows per block, row blocks,
// per-pass partial sums or null, arrival counters per row block (with
// partial sums), launch context; see k_stream_single).
using SingleFn = void (*)(MatDev, uint32_t, uint32_t, float*, uint32_t*, Fuse);

// Small-batch products (wal_gemm.hip).
//  * batched GEMV (vector ALUs), two launches: the first writes per-pass
//    partial sums P[pass][n][row] to the workspace (a wavefront takes
//    kGemvRows rows of one 4096-column pass for up to kGemvCols activation
//    columns, every decoded trit feeding all of them), and extra workgroups
//    of the same launch the low-rank reductions of every batch column per
//    4096-column chunk, zpart[chunk][n][term]; the second adds the passes and
//    the chunks in a fixed order, adds the low-rank term and stores Y.
//  * MFMA: the first blocks of the launch write the low-rank partials; every
//    other workgroup takes 128 rows by one kSliceCols-column slice for up to
//    32 activation columns on the matrix cores and writes its slice's partial
//    sums P[slice][n][row]; the same reduce kernel finishes Y.
// Large batches (prefill) run MFMA workgroups of 256 (fp16 scales) or 128
// rows by 64 activation columns over all columns (or an even share of them, split when the tiles
// alone would not fill the GPU) after a low-rank pre-pass; see PrefillShape.
constexpr uint32_t kGemvRows = 8;
constexpr uint32_t kGemvCols = 4;
constexpr uint32_t kZChunkCols = 4096;   // columns per low-rank partial (small batch)
// Single products: columns per low-rank partial, and the partials a streaming
// workgroup prefetches (more are added after the set-up barrier).
constexpr uint32_t kZSingleCols = 8192;
constexpr int kZSinglePrefetch = 4;
constexpr uint32_t kZTermsPerBlock = 16;
// Columns of one partial-sum slice of the MFMA small-batch kernel.
constexpr uint32_t kSliceCols = 1024;

// Workspace of the single and small-batch products: synchronisation words
// and arrival counters (kWsZeroBytes, zero before the first call), the
// low-rank partials, then partial sums.
struct GemmShape {
  uint32_t nt, passes, zc;   // n-tiles, batched GEMV passes, z chunks
  uint32_t slices;           // partial-sum planes of P: ceil(in / kSliceCols) >= passes
  uint64_t off_cnt, off_z, off_p, bytes;
};
GemmShape gemm_shape(const wal_info& f, uint32_t batch);
// Launchers (stream as hipStream_t); WAL_OK or WAL_ERR_DEVICE.
int launch_gemm_valu(const wal_info& f, const MatDev& d, uint32_t batch, void* ws, void* stream);
int launch_gemm_mfma(const wal_info& f, const MatDev& d, uint32_t batch, void* ws, void* stream);

// Prefill products: tiles of prefill_rows(scale format) rows x kPrefillCols
// activation rows (two 16-row tiles per wavefront with fp16 scales, one with
// fp24 scales, whose byte-wise loads need more registers).  A tile id names
// (row block, column chunk, K split); see k_prefill for the order of the ids
// and their mapping to workgroups.  K splits are made only while
// rblocks * chunks * nsplit < kPrefillTiles; their partial sums
// P[split][n][row] go to the workspace after the low-rank partials
// [zc][batch][terms] (zc column splits of zgroups groups, chosen so that the
// pre-pass runs about kZmmaWaves wavefronts, at most kZmmaMaxSplits: every
// consumer adds the zc partials).
constexpr uint32_t kPrefillWaves = 8;
constexpr uint32_t prefill_rows(uint32_t scale_fmt) { return kPrefillWaves * 16 * (scale_fmt == WAL_SCALE_FP16 ? 2 : 1); }
constexpr uint32_t kPrefillCols = 64;
constexpr uint32_t kPrefillTiles = 256;   // workgroups the GPU holds at once (1 per CU)
constexpr uint32_t kPrefillSweepGroups = 2;   // 128-column groups per sweep (a K split holds whole sweeps)
constexpr uint32_t kZmmaWaves = 1024;
constexpr uint32_t kZmmaMaxSplits = 8;
struct PrefillShape {
  uint32_t rblocks, chunks, nsplit, sweeps;   // sweeps of kPrefillSweepGroups groups over the whole K
  uint32_t cgw, per_xcd, tiles;               // chunks per id group, ids per XCD, padded ids
  uint32_t zc, zgroups;                       // low-rank partials per batch row, groups per partial
  uint64_t off_p, bytes;                      // workspace layout
};
PrefillShape prefill_shape(const wal_info& f, uint32_t batch);
int launch_gemm_prefill(const wal_info& f, const MatDev& d, uint32_t batch, void* ws, void* stream);

// Host helpers implemented in wal_host.cpp.
int check_info(const wal_info* info);

// Base-3 streaming kernels (wal_base3.hip), bf16 activations, by
// (scale format, k) class (4 * scale_fmt + index of k in {0, 2, 4, 8}) and
// whether they rotate x (WAL_X_ROT_H128), and the longest row range one of
// their workgroups takes.
GroupedFn base3_grouped_kernel(uint32_t cls, bool rot);
SingleFn base3_single_kernel(uint32_t cls, bool rot);
uint32_t base3_seg_rows();

}  // namespace wal
