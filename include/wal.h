/*
 * wal.h - C ABI of libwal: matrix-vector products taken directly from the
 * packed WAL ternary-hybrid weight format on AMD Instinct MI355X (gfx950).
 *
 * The operator is the one printed on the WAL-Ternary-8B model cards (Kazakh
 * card, section "Модель пішімі"; English card, section "Representation"):
 *
 *     y = W(x) = (alpha * T + beta * R) x + sum_p sum_r s_p[r] U_p[:, r] (V_p[:, r]^T x)
 *
 *   T    ternary base, entries in {-1, 0, +1} ("T3", strict ternary);
 *   R    exactly k signed residual sites per (row, group of 128 columns),
 *        k in {0, 2, 4, 8} ("exactly 8 signed residual sites per group of
 *        128 weights"; k0/k2/k4/k8 on the WAL-Ternary-27B-RC1 card,
 *        "Representation");
 *   alpha, beta  one scale per (row, group of 128 columns) (scale group 128:
 *        WAL2-Ternary-27B card, "Архитектура"), stored as fp16 or as a 24-bit
 *        float (the RC1 card's "24-bit float storage format decoded to FP32");
 *   U_p, V_p  binary {+1, -1} low-rank factors of up to 4 paths ("WALB2",
 *        two paths on the RC1 card), each path with fp16 per-rank scales s_p.
 *
 * No dense copy of W is ever formed: every kernel reads the packed planes.
 *
 * Blob layout (format version 1, little-endian), the byte-level reading of
 * the pages used by this library:
 *   header, 256 bytes:
 *     0 u32 magic 0x314C4157 ("WAL1")  4 u32 version = 1
 *     8 u32 out  12 u32 in  16 u32 k  20 u32 n_paths  24 u32 rank
 *     28 u32 trit_fmt  32 u32 scale_fmt  36 u32 row_stride
 *     40 u64 total_bytes  48 u64 off_codes  56 u64 off_sites  64 u64 off_alpha
 *     72 u64 off_beta  80 u64 off_V[4]  112 u64 off_U[4]  144 u64 off_s[4]
 *     176 u64 checksum = sum_i (i+1) * w_i mod 2^64 over the u32 words w_i
 *         that follow the header;  184..255 zero.
 *   planes, each at a multiple of 256 bytes, in the order
 *     codes [out][row_stride]
 *        2-bit:  row_stride = in/4; trit j of a row in bits 2(j%4)..2(j%4)+1
 *                of byte j/4; 0 -> 00, +1 -> 01, -1 -> 11 (10 is invalid;
 *                three of four codes used, WAL2-Ternary-27B card,
 *                "Что означает битность").
 *        base-3: five trits per byte (same section), packed continuously
 *                along the row: byte m = sum_{i<5} (t[5m+i] + 1) * 3^i;
 *                trits past `in` are zero; row_stride = ceil(in/5) rounded up
 *                to 16, pad bytes 0x79 (five zero trits); bytes > 242 invalid.
 *     sites [out][in/128][k]  (k > 0): bits 0-6 position in the group, bit 7
 *                set = negative sign; ascending, distinct positions.
 *     alpha [out][in/128], beta [out][in/128] (k > 0): fp16 (2 bytes) or fp24
 *                (the upper 3 bytes of the fp32 pattern, little-endian).
 *     per path p: V_p [rank][in/8] bits along `in`, U_p [out][ceil(rank/8)]
 *                bits along rank, LSB first, set bit = -1, pad bits zero;
 *                s_p [rank] fp16.
 *
 * Conventions for every call:
 *   - The caller allocates and owns every buffer.  Host pointers are used by
 *     the packing calls; device pointers (from hipMalloc or torch) by the
 *     product calls.  Packing and product calls allocate no memory, never
 *     synchronise a stream and keep no pointer after they return.  The one
 *     exception is wal_graph_create: it creates a HIP stream for the capture
 *     (destroyed before it returns), a graph, its executable form and a small
 *     host handle, all of which wal_graph_destroy frees.
 *   - Product calls enqueue work on `stream` (a hipStream_t; NULL = the
 *     default stream) and return.  y / Y is overwritten, never accumulated.
 *     x / X is read-only and must not overlap y / Y.
 *   - Every argument, shape, alignment and format check happens before any
 *     launch and returns a negative wal_status (fail-closed).  A failed
 *     launch returns WAL_ERR_DEVICE.  A device fault surfaces at the
 *     caller's next synchronisation of the stream.
 *   - Calls are reentrant; the library holds no mutable global state.
 */
#ifndef WAL_H
#define WAL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WAL_OK = 0,
  WAL_ERR_ARG = -1,         /* NULL pointer or value out of its domain      */
  WAL_ERR_SHAPE = -2,       /* in % 128 != 0, zero size, rank/paths limits  */
  WAL_ERR_CODE = -3,        /* invalid trit, site, sign or factor entry     */
  WAL_ERR_INEXACT = -4,     /* scale not exactly representable when packing */
  WAL_ERR_BUFFER = -5,      /* buffer too small                              */
  WAL_ERR_ALIGN = -6,       /* device pointer misaligned                    */
  WAL_ERR_FORMAT = -7,      /* bad magic, version, layout or checksum       */
  WAL_ERR_DEVICE = -8,      /* a HIP call or kernel launch failed           */
  WAL_ERR_UNSUPPORTED = -9  /* valid input that this build does not handle  */
} wal_status;

enum { WAL_TRIT_2BIT = 0, WAL_TRIT_BASE3 = 1 };
enum { WAL_SCALE_FP16 = 0, WAL_SCALE_FP24 = 1 };
enum { WAL_X_F32 = 0, WAL_X_BF16 = 1 };
/* Flag OR-ed into the x_dtype of wal_gemv, wal_gemv_noalloc and the grouped
 * plans (hence chains and graphs): the blob was stored rotated (WAL2-Ternary-
 * 27B card, "Архитектура": W' = W R, R the normalised H128 of
 * wal_rotate_h128, one block per 128-column group), so the product takes the
 * rotated activations, y = W'(R x).  The launch rotates x itself, with
 * wal_rotate_h128's arithmetic and rounding (the result keeps x's type), so
 * the output equals wal_rotate_h128 followed by the plain product bit for
 * bit; x itself is not written.  The batched calls (wal_gemm_small,
 * wal_gemm_prefill) return WAL_ERR_UNSUPPORTED with it: rotate X once with
 * wal_rotate_h128 for the whole batch. */
#define WAL_X_ROT_H128 16
enum { WAL_GEMM_AUTO = 0, WAL_GEMM_VALU = 1, WAL_GEMM_MFMA = 2 };

#define WAL_MAX_PATHS 4
#define WAL_MAX_RANK 64
#define WAL_HEADER_BYTES 256
#define WAL_MAX_BATCH 32
#define WAL_MAX_PREFILL_BATCH 16384

/* Shape and storage choice of one matrix. */
typedef struct {
  uint32_t out, in;        /* W is out x in; in must be a multiple of 128   */
  uint32_t k;              /* sites per group: 0, 2, 4 or 8                 */
  uint32_t n_paths, rank;  /* binary low-rank paths (0..4), rank (1..64)    */
  uint32_t trit_fmt;       /* WAL_TRIT_2BIT or WAL_TRIT_BASE3               */
  uint32_t scale_fmt;      /* WAL_SCALE_FP16 or WAL_SCALE_FP24 (alpha, beta) */
} wal_desc;

/* Host-side view of one blob: its descriptor and plane offsets. */
typedef struct {
  wal_desc d;
  uint32_t row_stride;     /* bytes per row of the code plane               */
  uint32_t groups;         /* in / 128                                      */
  uint64_t total_bytes;    /* size of the blob                              */
  uint64_t off_codes, off_sites, off_alpha, off_beta;
  uint64_t off_V[WAL_MAX_PATHS], off_U[WAL_MAX_PATHS], off_s[WAL_MAX_PATHS];
  uint64_t algorithmic_bytes; /* plane bytes a product reads (no header,
                                 alignment or base-3 row padding)           */
} wal_info;

#define WAL_MAX_CLASSES 16

/* Launch summary of a grouped plan (filled by wal_grouped_plan).  Matrices
 * are grouped by kernel class, class id = 8 * trit_fmt + 4 * scale_fmt +
 * index of k in {0, 2, 4, 8}; each class present gets one streaming launch
 * over its own split of rows into class_grid[c] workgroups.  The low-rank
 * reductions run as n_zjobs jobs of zjob_terms terms (4 when that makes at
 * most 64 jobs, else 16) over one 4096-column chunk each. */
typedef struct {
  uint32_t n;              /* matrices                                      */
  uint32_t n_classes;      /* classes present (streaming launches)          */
  uint32_t n_segs;         /* (matrix, row range) segments, all classes     */
  uint32_t n_zjobs;        /* workgroups of the low-rank V^T x pre-pass     */
  uint32_t x_dtype;        /* as passed to wal_grouped_plan, flags included */
  uint32_t zjob_terms;     /* low-rank terms per job (4 or 16)             */
  uint32_t rows_per_batch; /* rows a wavefront reduces at once              */
  uint32_t grid;           /* largest class grid                           */
  uint64_t plan_bytes;     /* bytes of the plan blob                        */
  uint64_t algorithmic_bytes; /* sum of the matrices' algorithmic bytes     */
  uint64_t off_descs, off_zjobs;              /* plan offsets               */
  uint32_t class_id[WAL_MAX_CLASSES];
  uint32_t class_grid[WAL_MAX_CLASSES];
  uint64_t class_blockseg[WAL_MAX_CLASSES];   /* plan offsets per class     */
  uint64_t class_segs[WAL_MAX_CLASSES];
  void* sync_dev;          /* the workspace's synchronisation words (its
                              start), or NULL when the plan has no low-rank
                              paths and no split matrices                  */
} wal_grouped_info;

/* Human-readable name of a status code (static string, never NULL). */
const char* wal_status_str(int status);

/* Layout of a blob for `desc`: fills *info (offsets, total and algorithmic
 * bytes).  Defined by the layout above.  Errors: ARG, SHAPE. */
int wal_packed_size(const wal_desc* desc, wal_info* info);

/* Pack logical arrays (host memory) into a blob at dst (host, dst_bytes >=
 * info.total_bytes).  Arrays, all row-major:
 *   T          int8   [out][in]        values in {-1, 0, +1}
 *   site_pos   uint8  [out][in/128][k] ascending, distinct, < 128  (k > 0)
 *   site_sign  int8   [out][in/128][k] values in {-1, +1}          (k > 0)
 *   alpha      float  [out][in/128]
 *   beta       float  [out][in/128]                                (k > 0)
 *   U          int8   [n_paths][out][rank]   values in {-1, +1}
 *   V          int8   [n_paths][in][rank]    values in {-1, +1}
 *   s          float  [n_paths][rank]
 * Pointers of absent parts (k == 0: sites, beta; n_paths == 0: U, V, s) may
 * be NULL.  A scale that its storage format cannot hold exactly is rejected
 * (WAL_ERR_INEXACT); nothing is rounded.  On success *info (if not NULL)
 * describes the blob.  Errors: ARG, SHAPE, CODE, INEXACT, BUFFER. */
int wal_pack(const wal_desc* desc, const int8_t* T, const uint8_t* site_pos,
             const int8_t* site_sign, const float* alpha, const float* beta,
             const int8_t* U, const int8_t* V, const float* s,
             void* dst, size_t dst_bytes, wal_info* info);

/* Parse and check a blob's header and layout (not its planes).  With
 * wal_verify and wal_unpack below, this is the fail-closed check of a packed
 * cache before use (WAL-Ternary-8B cards, "Install" / "Орнату": the cache of
 * packed ternary symbols, sparse positions and signs and fp16 scales is
 * verified fail-closed).  Errors: ARG, BUFFER, FORMAT. */
int wal_inspect(const void* blob, size_t bytes, wal_info* info);

/* Full check of a host blob: header, layout, checksum and every stored code
 * (2-bit 10, base-3 byte > 242 or bad padding, unsorted or repeated sites,
 * non-zero pad bits).  Errors: ARG, BUFFER, FORMAT, CODE. */
int wal_verify(const void* blob, size_t bytes);

/* Unpack a verified host blob into logical arrays with the shapes of
 * wal_pack (outputs of absent parts may be NULL).
 * Errors: those of wal_verify. */
int wal_unpack(const void* blob, size_t bytes, int8_t* T, uint8_t* site_pos,
               int8_t* site_sign, float* alpha, float* beta, int8_t* U,
               int8_t* V, float* s);

/* Device workspace that wal_gemv and wal_gemm_small need for a blob and
 * batch.  The WALB2 term sum_r U_r (V_r^T x) of the operator (WAL-Ternary-8B
 * cards, "Representation") needs every V_r^T x complete before U expands it,
 * so its partial sums live in device memory between the two steps; the
 * small-batch kernels also keep partial products there.  Contents, each part
 * padded to 256 bytes:
 *   WAL_WS_ZERO_BYTES that must be zero before the workspace's first use
 *     (hipMemset, torch.zeros) and that every call leaves as it found them,
 *     except two things: the epoch words, which count the calls made on the
 *     workspace (a call's low-rank partials carry a tag derived from it, so
 *     that no call takes another's partials for its own), and the u32 word
 *     WAL_SYNC_FALLBACK_WORD, a diagnostic count: a workgroup adds one when
 *     its bounded wait for the low-rank terms gives up and it computes them
 *     itself (outputs stay exact; the caller may read and clear the word).
 *     The region has the same size and place for every blob, so one
 *     workspace serves products of any shape in turn.  It holds
 *     WAL_SYNC_BYTES of synchronisation words (u32; the workgroups of one
 *     launch coordinate through them, see wal_gemv), then one arrival
 *     counter (u32) per 16 rows of a split product, for up to
 *     WAL_MAX_ROW_BLOCKS of them (a product with more rows runs its passes
 *     in sequence);
 *   the per-path reductions z_p = diag(s_p) V_p^T X: the small-batch
 *     kernels' per 4096-column chunk [chunks][batch][n_paths * rank] (fp32),
 *     or wal_gemv's per 8192-column chunk [chunks][n_paths * rank] (fp32
 *     value and u32 tag), whichever is larger;
 *   the small-batch kernels' partial sums per 1024-column slice
 *     [ceil(in / 1024)][batch][out] (fp32).
 * wal_gemv uses the last part only for matrices wider than one pass.
 * Errors: ARG, SHAPE, FORMAT. */
#define WAL_SYNC_BYTES 4352
#define WAL_SYNC_FALLBACK_WORD 0
#define WAL_MAX_ROW_BLOCKS 4096
#define WAL_WS_ZERO_BYTES (WAL_SYNC_BYTES + 4 * WAL_MAX_ROW_BLOCKS)
int wal_workspace_size(const wal_info* info, uint32_t batch, size_t* bytes);

/* y = W(x) for one matrix, batch 1 (WAL-Ternary-8B cards, "Representation":
 * the ternary-hybrid product with its binary low-rank paths), one launch:
 * its first workgroups compute the low-rank terms V^T x, the others stream
 * the packed planes and wait for those terms (bounded, through the
 * workspace's synchronisation words) only when they store their rows; a
 * workgroup whose wait gives up computes the terms itself.  A matrix wider than one pass (4096 columns,
 * 5120 for base-3 codes) has its passes in separate workgroups when the
 * workspace is wal_workspace_size(info, 1) bytes; the workgroup that
 * completes a 16-row group adds its passes in pass order.
 *   info   host view of the blob (from wal_inspect / wal_pack)
 *   W_dev  the blob in device memory, 256-byte aligned
 *   x_dev  [in] activations, fp32 or bf16 (x_dtype), 16-byte aligned
 *   y_dev  [out] fp32 output, 4-byte aligned, overwritten
 *   ws_dev workspace of wal_workspace_size(info, 1) bytes, 16-byte aligned,
 *          disjoint from x and y, its first WAL_WS_ZERO_BYTES zero before
 *          its first use (may be NULL for a blob without paths)
 * Errors: ARG, SHAPE, ALIGN, BUFFER, UNSUPPORTED, DEVICE. */
int wal_gemv(const wal_info* info, const void* W_dev, const void* x_dev, int x_dtype,
             float* y_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* y = W(x) as wal_gemv, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the workspace is a file-scope device array of
 * WAL_NOALLOC_SCRATCH_BYTES (4 MiB) that each GPU holds from the library's
 * first use until the process ends; the call itself allocates nothing.
 * Arguments as for wal_gemv.  A blob whose low-rank partials exceed the
 * scratch returns WAL_ERR_BUFFER (4 bytes per term and 4096-column chunk:
 * only past 16 million columns at the maximum of 256 terms); a wide matrix
 * whose per-pass partial sums do not fit
 * runs its passes in sequence instead of splitting them.  Every call on a
 * GPU shares that GPU's scratch: calls that overlap on one GPU (several
 * streams or threads) race and must be ordered by the caller.
 * Errors: those of wal_gemv, BUFFER. */
#define WAL_NOALLOC_SCRATCH_BYTES (4u << 20)
int wal_gemv_noalloc(const wal_info* info, const void* W_dev, const void* x_dev, int x_dtype, float* y_dev,
                     void* stream);

/* Y = X W^T for a small batch (F.linear convention): row n of Y is W(x_n)
 * with x_n row n of X (WAL-Ternary-8B cards, "Representation").
 *   X_dev  [batch][ldx] activations (bf16 or fp32), ldx >= in, ldx*elem % 16 == 0,
 *          ((batch - 1) * ldx + in) * elem < 2^31 bytes (else WAL_ERR_SHAPE)
 *   Y_dev  [batch][ldy] fp32 outputs, ldy >= out; columns past out untouched
 *   batch  1..WAL_MAX_BATCH
 *   mode   WAL_GEMM_VALU (batched GEMV: one decode of a row feeds every batch
 *          column on the vector ALUs), WAL_GEMM_MFMA (trits decoded to bf16
 *          operands of matrix-core MFMA, alpha / beta applied per group in
 *          fp32) or WAL_GEMM_AUTO (MFMA from a measured crossover batch on,
 *          the batched GEMV below it, the single-product path at batch 1).
 *          Both batched kernels take bf16 X and 2-bit codes; fp32 X or
 *          base-3 codes run one wal_gemv per row with WAL_GEMM_VALU / AUTO,
 *          and WAL_GEMM_MFMA returns WAL_ERR_UNSUPPORTED for them.
 *   ws_dev wal_workspace_size(info, batch) bytes, 16-byte aligned, disjoint
 *          from X and Y; its first WAL_WS_ZERO_BYTES zero before its first
 *          use (the single-product path uses them), the rest need not be
 * Calls that share a workspace must be ordered (one stream).
 * Errors: ARG, SHAPE, ALIGN, BUFFER, UNSUPPORTED, DEVICE. */
int wal_gemm_small(const wal_info* info, const void* W_dev, const void* X_dev, int x_dtype,
                   uint32_t batch, uint32_t ldx, float* Y_dev, uint32_t ldy, int mode,
                   void* ws_dev, size_t ws_bytes, void* stream);

/* Device workspace that wal_gemm_prefill needs for a blob and batch
 * (1..WAL_MAX_PREFILL_BATCH): the low-rank partials [zc][batch][n_paths *
 * rank], one per column split of the pre-pass (zc splits of whole 128-column
 * groups, as many as bring the pre-pass to about 1024 wavefronts of 16 batch
 * rows x 16 terms, at most 8) and, when the product is split along K (few
 * output tiles),
 * the per-split partial sums [splits][batch][out] (fp32), each part padded to
 * 256 bytes.  0 for a blob without paths that is not split.
 * Errors: ARG, SHAPE, FORMAT. */
int wal_prefill_workspace_size(const wal_info* info, uint32_t batch, size_t* bytes);

/* Y = X W^T for a prefill-size batch (F.linear convention; WAL-Ternary-8B
 * cards, "Representation", and the pages' note that batched packed products
 * were left unoptimised): trits decoded to bf16 operands of matrix-core MFMA
 * tiles of 128 rows x 32 activation rows, alpha / beta applied per group in
 * fp32, the low-rank term added from a pre-pass.
 *   X_dev  [batch][ldx] bf16 activations, ldx >= in, ldx * 2 % 16 == 0,
 *          (batch - 1) * ldx + in < 2^30 elements
 *   Y_dev  [batch][ldy] fp32 outputs, ldy >= out; columns past out untouched
 *   batch  1..WAL_MAX_PREFILL_BATCH (any batch works; from a few hundred rows
 *          on, the tiles alone fill the GPU and nothing is split)
 *   ws_dev wal_prefill_workspace_size(info, batch) bytes, 16-byte aligned,
 *          disjoint from X and Y (may be NULL when that size is 0)
 * fp32 X and base-3 codes return WAL_ERR_UNSUPPORTED.  Every sum runs in a
 * fixed order: results do not depend on timing.  Calls that share a
 * workspace must be ordered (one stream).
 * Errors: ARG, SHAPE, ALIGN, BUFFER, UNSUPPORTED, DEVICE. */
int wal_gemm_prefill(const wal_info* info, const void* W_dev, const void* X_dev, int x_dtype,
                     uint32_t batch, uint32_t ldx, float* Y_dev, uint32_t ldy,
                     void* ws_dev, size_t ws_bytes, void* stream);

/* Grouped products y_i = W_i(x_i), i < n, in one pass over all matrices
 * (e.g. the 252 body matrices of a 36-layer model, all of which run straight
 * from the packed form: WAL-Ternary-8B cards, "Модель пішімі" /
 * "Representation", 252/252 body matrices).  Two steps:
 *   1. wal_grouped_plan writes a plan blob into plan_host (host memory of
 *      plan_bytes, see wal_grouped_plan_size) describing every matrix (device
 *      pointers of its planes, x_i, y_i, its workspace slot) and, for each
 *      (scale format, k) class, a split of the class's rows into `grid`
 *      contiguous ranges of equal packed bytes, one per workgroup of that
 *      class's streaming launch.  grid = 0 asks for the number of
 *      workgroups the current device holds at once (a HIP query; the other
 *      steps of planning are host-only), capped at one per 16 rows of a
 *      pass.  A class with fewer 16-row groups than workgroups runs the
 *      passes of its wider matrices in separate workgroups (their partial
 *      sums in the workspace, added in pass order by the workgroup that
 *      completes a 16-row group).
 *   2. The caller copies the plan blob into device memory (plan_dev, 16-byte
 *      aligned) and calls wal_gemv_grouped, as often as it likes while the
 *      pointers stay valid.  A call's first streaming launch computes the
 *      low-rank terms in its first workgroups, and the streaming workgroups
 *      wait for them (bounded) only when they store their rows; a
 *      workgroup whose wait gives up computes them itself.
 * All matrices share x_dtype (with WAL_X_ROT_H128 every matrix of the plan
 * takes its own x rotated); base-3 matrices need bf16 activations
 * (WAL_ERR_UNSUPPORTED otherwise).  ws_dev must hold
 * wal_grouped_plan_size's ws_bytes, 16-byte aligned (NULL when that is 0).
 * When the plan has low-rank paths or split matrices, the workspace starts
 * with the zero region of wal_workspace_size (WAL_WS_ZERO_BYTES, zero before
 * its first use, left so by every call except the diagnostic count
 * WAL_SYNC_FALLBACK_WORD and the epoch words); one workspace may serve any
 * number of plans, products and shapes in turn.  Calls that share a
 * workspace must be ordered (one stream).
 * Errors: ARG, SHAPE, ALIGN, BUFFER, UNSUPPORTED, DEVICE. */
int wal_grouped_plan_size(uint32_t n, const wal_info* infos, uint32_t grid, int x_dtype,
                          size_t* plan_bytes, size_t* ws_bytes);
int wal_grouped_plan(uint32_t n, const wal_info* infos, const void* const* W_dev,
                     const void* const* x_dev, int x_dtype, float* const* y_dev,
                     void* ws_dev, size_t ws_bytes, uint32_t grid, void* plan_host,
                     size_t plan_bytes, wal_grouped_info* ginfo);
int wal_gemv_grouped(const wal_grouped_info* ginfo, const void* plan_dev, void* stream);

/* The two phases of wal_gemv_grouped, for callers that schedule or time them
 * apart: WAL_PHASE_LOWRANK launches the low-rank pre-pass on its own (z_p of
 * every matrix into the workspace given to wal_grouped_plan),
 * WAL_PHASE_STREAM the streaming launches (one per class), which then read
 * those z_p without waiting; the pre-pass of a call must precede its
 * streaming phase on the stream.  WAL_PHASE_ALL is wal_gemv_grouped (the
 * pre-pass inside the first streaming launch).
 * Errors: those of wal_gemv_grouped; ARG for an empty or unknown mask. */
enum { WAL_PHASE_LOWRANK = 1, WAL_PHASE_STREAM = 2, WAL_PHASE_ALL = 3 };
int wal_gemv_grouped_phases(const wal_grouped_info* ginfo, const void* plan_dev, int phases,
                            void* stream);

/* INT4/g128 packed matrices: the LM head of the WAL-Ternary-8B cards (Kazakh
 * card, "Модель пішімі", and the English card list it as INT4/g128; nothing
 * more is printed).  This repository's reading: W[v][j] = s[v][j / 128] *
 * q[v][j] with q a signed 4-bit integer in [-8, 7] and one fp16 scale per 128
 * consecutive columns (symmetric, no zero point).  Layout of a [V][in] matrix
 * (in a multiple of 128):
 *   codes  [V][in / 2] bytes, element 2i in the low nibble of byte i, 2i + 1
 *          in the high nibble, two's-complement nibbles
 *   scales [V][in / 128] fp16, little-endian, right after the codes
 * wal_int4_size: bytes of the layout (V * in above 2^40: WAL_ERR_SHAPE).
 *   Errors: ARG, SHAPE.
 * wal_int4_pack: q int8 [V][in], s float [V][in / 128] (host) -> dst (host).
 *   A code outside [-8, 7] (WAL_ERR_CODE) or a scale fp16 cannot hold exactly
 *   (WAL_ERR_INEXACT) is rejected before anything is written.
 *   Errors: ARG, SHAPE, CODE, INEXACT, BUFFER.
 * wal_int4_unpack: the inverse (q or s may be NULL).  Errors: ARG, SHAPE, BUFFER.
 * wal_int4_gemv: y[v] = sum_j W[v][j] x[j] on the GPU, one matrix, batch 1.
 *   W_dev  the layout in device memory, 256-byte aligned
 *   x_dev  [in] bf16, 16-byte aligned (fp32 x: WAL_ERR_UNSUPPORTED)
 *   y_dev  [V] fp32, overwritten; must not overlap W or x (WAL_ERR_ARG)
 *   The packed matrix must be under 2^31 bytes (else WAL_ERR_SHAPE).
 *   Errors: ARG, SHAPE, ALIGN, UNSUPPORTED, DEVICE. */
int wal_int4_size(uint32_t V, uint32_t in, size_t* bytes);
int wal_int4_pack(uint32_t V, uint32_t in, const int8_t* q, const float* s, void* dst, size_t dst_bytes);
int wal_int4_unpack(uint32_t V, uint32_t in, const void* src, size_t src_bytes, int8_t* q, float* s);
int wal_int4_gemv(const void* W_dev, uint32_t V, uint32_t in, const void* x_dev, int x_dtype, float* y_dev,
                  void* stream);

/* INT3/g128 packed matrices: the embedding of the WAL-Ternary-8B cards (listed
 * as INT3/g128; nothing more is printed).  This repository's reading:
 * E[v][j] = s[v][j / 128] * q[v][j], q a signed 3-bit integer in [-4, 3], one
 * fp16 scale per 128 consecutive columns.  Layout of a [V][in] matrix:
 *   codes  [V][in * 3 / 8] bytes: row v's codes as one bit stream, element j
 *          at stream bits 3 j .. 3 j + 2 (stream bit b = bit b % 8 of byte
 *          b / 8), two's-complement codes
 *   scales [V][in / 128] fp16, little-endian, right after the codes
 * wal_int3_size / wal_int3_pack / wal_int3_unpack: as the INT4 functions,
 * with codes in [-4, 3].
 * wal_embed_rows: out[i][:] = row ids[i] of an INT3 (bits = 3) or INT4/g128
 * (bits = 4) matrix, decoded on the GPU: the embedding lookup of a batch of
 * tokens.  Each value is s * q, exact in fp32; bf16 output rounds it to
 * nearest even.
 *   W_dev    the matrix in device memory, 256-byte aligned
 *   ids_dev  [n] int32 row indices (device); an index outside [0, V) gives a
 *            row of zeros
 *   out_dev  [n][ldo] fp32 or bf16 (out_dtype), 16-byte aligned rows, ldo >= in;
 *            columns past `in` untouched
 *   The packed matrix must be under 2^32 bytes and n at most 2^31 - 1 (else
 *   WAL_ERR_SHAPE); out must not overlap W or ids (WAL_ERR_ARG).
 *   Errors: ARG, SHAPE, ALIGN, DEVICE. */
int wal_int3_size(uint32_t V, uint32_t in, size_t* bytes);
int wal_int3_pack(uint32_t V, uint32_t in, const int8_t* q, const float* s, void* dst, size_t dst_bytes);
int wal_int3_unpack(uint32_t V, uint32_t in, const void* src, size_t src_bytes, int8_t* q, float* s);
int wal_embed_rows(const void* W_dev, int bits, uint32_t V, uint32_t in, const int32_t* ids_dev, uint32_t n,
                   void* out_dev, int out_dtype, uint32_t ldo, void* stream);

/* wal_embed_rows_mixed: the embedding of the WAL-Ternary-27B-RC1 card
 * (section "Representation": three quarters of the rows INT3, a selected
 * quarter INT4).  This repository's reading: an INT3/g128 table [V3][in], an
 * INT4/g128 table [V4][in] (layouts above) and a row map [V]; vocabulary row
 * v is row m = map[v] of the INT3 table when m >= 0, else row -1 - m of the
 * INT4 table.  out[i][:] = vocabulary row ids[i], decoded as wal_embed_rows
 * does.
 *   W3_dev, W4_dev  the two tables in device memory, 256-byte aligned
 *   map_dev         [V] int32 (device); an entry outside its table gives a
 *                   row of zeros
 *   ids_dev         [n] int32 (device); an id outside [0, V) gives a row of
 *                   zeros
 *   out_dev, ldo, out_dtype  as for wal_embed_rows
 *   Each table must be under 2^32 bytes and n at most 2^31 - 1 (else
 *   WAL_ERR_SHAPE); out must not overlap the tables, the map or ids
 *   (WAL_ERR_ARG).
 *   Errors: ARG, SHAPE, ALIGN, DEVICE. */
int wal_embed_rows_mixed(const void* W3_dev, uint32_t V3, const void* W4_dev, uint32_t V4, uint32_t in,
                         const int32_t* map_dev, uint32_t V, const int32_t* ids_dev, uint32_t n, void* out_dev,
                         int out_dtype, uint32_t ldo, void* stream);

/* INT5/g128 packed matrices: the LM head of the WAL-Ternary-27B-RC1 card
 * (section "Representation" lists it as packed INT5; nothing more is
 * printed).  This repository's reading, in line with the other cards'
 * symmetric INT4/g128 head: W[v][j] = s[v][j / 128] * q[v][j], q a signed
 * 5-bit integer in [-16, 15], one fp16 scale per 128 columns, five bits per
 * weight with no padding.  Layout of a [V][in] matrix (in a multiple of 128):
 *   codes  [V][in * 5 / 8] bytes: row v's codes as one bit stream, element j
 *          at stream bits 5 j .. 5 j + 4 (stream bit b = bit b % 8 of byte
 *          b / 8), two's-complement codes
 *   scales [V][in / 128] fp16, little-endian, right after the codes
 * wal_int5_size / wal_int5_pack / wal_int5_unpack / wal_int5_gemv: as the
 * INT4 functions, with codes in [-16, 15]. */
int wal_int5_size(uint32_t V, uint32_t in, size_t* bytes);
int wal_int5_pack(uint32_t V, uint32_t in, const int8_t* q, const float* s, void* dst, size_t dst_bytes);
int wal_int5_unpack(uint32_t V, uint32_t in, const void* src, size_t src_bytes, int8_t* q, float* s);
int wal_int5_gemv(const void* W_dev, uint32_t V, uint32_t in, const void* x_dev, int x_dtype, float* y_dev,
                  void* stream);

/* The normalised Hadamard-128 rotation of activations (WAL2-Ternary-27B card,
 * "Архитектура": the packed weights are rotated by a normalised H128 with
 * sign_mode identity, so a product of such a blob takes the rotated x):
 *     out[r][128 g + i] = sum_j H[i][j] x[r][128 g + j] / sqrt(128)
 * with H Sylvester's Hadamard matrix, H[i][j] = (-1)^popcount(i & j).
 *   x_dev    [rows][ldx] bf16 or fp32 (x_dtype), 16-byte aligned rows
 *   in       columns, a multiple of 128 (else WAL_ERR_SHAPE)
 *   out_dev  [rows][ldo] bf16 or fp32 (out_dtype), 16-byte aligned rows;
 *            columns past `in` untouched.  out may be x itself (same type
 *            and pitch: in place); any other overlap is rejected
 * Arithmetic: bf16 input as the product X H on the matrix cores (exact
 * bf16 operands, fp32 sums), fp32 input as fp32 butterflies; then the
 * multiply by fp32(1/sqrt(128)), and bf16 output rounds to nearest even.
 * The products that rotate x themselves (WAL_X_ROT_H128) use the same
 * arithmetic.
 * Errors: ARG, SHAPE, ALIGN, DEVICE. */
int wal_rotate_h128(const void* x_dev, int x_dtype, uint32_t rows, uint32_t in, uint32_t ldx,
                    void* out_dev, int out_dtype, uint32_t ldo, void* stream);

/* A decode step as a chain of grouped products that depend on each other
 * (the 8B cards time their decode step with a captured graph, "Жылдамдық пен
 * жад" / speed and memory table): product
 * i + 1 starts only after product i has finished, as when matrices that
 * share an input (q|k|v, gate|up) form one grouped product and the next
 * product reads the previous one's output.
 *
 * wal_gemv_grouped_seq launches the n grouped products in order on `stream`
 * (plans_dev[i] as for wal_gemv_grouped with ginfos[i]).
 * Errors: those of wal_gemv_grouped, for the first product that fails (the
 * products before it are already enqueued). */
int wal_gemv_grouped_seq(uint32_t n, const wal_grouped_info* ginfos, const void* const* plans_dev,
                         void* stream);

/* The same chain captured once into a HIP graph and replayed with one call.
 * wal_graph_create captures the n grouped products (on a private stream of
 * default priority, which it destroys) and instantiates the graph; the
 * handle owns the graph.  Every buffer the plans name (plans, weights, x, y,
 * workspaces) must stay allocated while the handle exists; their contents may
 * change between launches (a replay reads x as it is then).
 * wal_graph_launch enqueues one replay on `stream`, after the work already
 * there.  wal_graph_destroy frees the graph (NULL is accepted).  The graph
 * holds only kernel launches: no memset or copy nodes.
 * Errors: ARG (n == 0, NULL arguments), those of wal_gemv_grouped found while
 * capturing (nothing is created then), DEVICE. */
typedef struct wal_graph wal_graph;
int wal_graph_create(uint32_t n, const wal_grouped_info* ginfos, const void* const* plans_dev,
                     wal_graph** graph);
int wal_graph_launch(const wal_graph* graph, void* stream);
int wal_graph_destroy(wal_graph* graph);

#ifdef __cplusplus
}
#endif
#endif /* WAL_H */
