/*
 * sk_gemm.h -- Stream-K dense GEMM for one AMD Instinct MI355X (gfx950).
 *
 * Computes C = alpha * A * B + beta * C (the GEMM definition of the Stream-K
 * page, "Stream-K: Work-centric Parallel Decomposition for Dense
 * Matrix-Matrix Multiplication on the GPU", section 3 background) with the
 * work-centric decomposition of that page's section 4 (Algorithm 5) and the
 * "two-tile Stream-K + data-parallel" hybrid of its section 5.2, optionally
 * with threadblock-level ABFT checksums ("Anatomy of High-Performance GEMM
 * with Online Fault Tolerance on GPUs", threadblock-level scheme, Figs. 5-7;
 * the column and row encodings of each tile row of A and tile column of B
 * are formed once per call by a separate kernel, and the MAC loop keeps
 * only the checksum updates).
 * Matrix-vector products (m or n = 1) and a few vectors at once (up to 16,
 * fp16/bf16 up to 8) take the even split of "KBLAS: An Optimized Library for
 * Dense Matrix-Vector Multiplication on GPU Accelerators" (section 6.2)
 * instead of output tiles (SK_SCHED_GEMV_SPLIT).
 *
 * Conventions shared by every entry point:
 *  - A is m x k, B is k x n, C is m x n.  Storage order of A and B is given by
 *    sk_layout; C is always row-major (element (i, j) at C[i * ldc + j]).
 *    Leading dimensions are in elements.  Row-major A needs lda >= k,
 *    column-major A needs lda >= m; row-major B needs ldb >= n, column-major
 *    B needs ldb >= k; ldc >= n.  A column-major C (element (i, j) at
 *    C[j * ldc + i]) is the row-major n x m matrix C^T = B^T A^T: call with
 *    m and n swapped, B's pointer and leading dimension as the first operand
 *    and A's as the second, and each operand's storage order flipped (B
 *    column-major becomes a row-major first operand, and so on).
 *  - A, B and C are device pointers owned by the caller; the library never
 *    frees them.  A and B are read only; C is read only when beta != 0.
 *  - Calls are asynchronous: work is enqueued on `stream` (0 = the default
 *    stream) and the call returns; results are valid once the stream has been
 *    synchronised.  No host synchronisation happens inside a call, except
 *    that the first call on a (device, stream) pair allocates the library's
 *    workspace (partial tiles and flags for the cross-workgroup fixup).
 *  - Two host threads must not issue calls on the same stream at the same
 *    time (they would share one workspace).
 *  - Return value: SK_OK (0) or a negative sk_status.  No exception crosses
 *    this interface.  Errors found on the device (a fixup wait that timed
 *    out, the result of that call being wrong) are reported once: by the
 *    next sk_gemm / sk_gemm_ex call on the device that starts after the
 *    kernel wrote its error word (that call returns SK_ERR_FIXUP_TIMEOUT and
 *    launches nothing), or by sk_device_status(), whichever comes first.
 */
#ifndef SK_GEMM_H
#define SK_GEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  SK_F32: fp32 in and out, fp32 accumulation (SGEMM).
 * SK_F16 / SK_BF16: fp16 / bf16 in and out, fp32 accumulation (HGEMM);
 * alpha and beta are applied in fp32 and the result is rounded once to the
 * output type (round to nearest even). */
typedef enum { SK_F32 = 0, SK_F16 = 1, SK_BF16 = 2 } sk_dtype;

/* Storage order of A and B ("ROW": the second index is contiguous).
 * SK_A_ROW_B_COL keeps both operands contiguous along k.  Operands are read
 * in place when the base is 16-byte aligned, the leading dimension a
 * multiple of 16 bytes, and: for a k-contiguous operand, k a multiple of 16
 * bytes of elements; fp32, either order; fp16/bf16 A stored m-contiguous
 * (column-major) or B stored n-contiguous (row-major): m (A) or n (B) a
 * multiple of 8, 2 (k + 64) ld + 1024 below 2^31 - 1 (bytes) and the LARGE
 * or SMALL tile instance (transposed in LDS; NARROW reads k-contiguous
 * operands only).  Any other operand is repacked into a k-contiguous copy
 * first (see sk_gemm_ex). */
typedef enum {
  SK_A_ROW_B_ROW = 0,
  SK_A_ROW_B_COL = 1,
  SK_A_COL_B_ROW = 2,
  SK_A_COL_B_COL = 3
} sk_layout;

typedef enum {
  SK_OK = 0,
  SK_ERR_INVALID_ARG = -1,   /* negative size, leading dimension too small, NULL pointer with nonzero size, bad enum */
  SK_ERR_UNSUPPORTED = -2,   /* combination the library does not implement (e.g. an operand row over 8 MiB) */
  SK_ERR_NO_MEMORY = -3,     /* workspace allocation failed */
  SK_ERR_HIP = -4,           /* a HIP runtime call or kernel launch failed; sk_last_hip_error() has the text */
  SK_ERR_FIXUP_TIMEOUT = -5, /* device: a workgroup gave up waiting for a peer's partial tile */
  SK_ERR_NO_DEVICE = -6,     /* no usable gfx950 device */
  SK_ERR_TOO_LARGE = -7      /* sk_gemm_noalloc: the call needs more scratch than it holds */
} sk_status;

/* Work decompositions.  The first four are the Stream-K page's, with tiles in
 * linear m -> n order:
 *  SK_SCHED_DP        data-parallel (Algorithm 2), persistent over the slots.
 *  SK_SCHED_SK_BASIC  basic Stream-K (Algorithm 5) over all tiles.
 *  SK_SCHED_SK_HYBRID2 "two-tile Stream-K + data-parallel" (section 5.2).
 *  SK_SCHED_SK_HYBRID1 "data-parallel + one-tile Stream-K" (section 5.2).
 * SK_SCHED_XCD_ALIGNED is this library's MI355X form of the same work-centric
 * split: the Stream-K region (all tiles when there are fewer than the slots,
 * else one full wave plus the leftover tiles, as in the two-tile hybrid) is
 * split in quanta of ipt / D iterations so that the workgroups resident on
 * one XCD run at equal k offsets on a compact block of tiles (they then share
 * the A and B slices they read in that XCD's L2), and data-parallel tiles are
 * dealt in compact per-XCD blocks.  With no leftover tiles it is
 * data-parallel in that XCD-aware order.
 *  SK_SCHED_GEMV_SPLIT matrix-vector products (m == 1 or n == 1), the work
 *                     split evenly over the workgroups (the KBLAS page's
 *                     block-row split, section 6.2; Stream-K's work-centric
 *                     idea at the level of dot products).  With the matrix
 *                     operand k-contiguous (16-byte aligned base and rows)
 *                     and the vector contiguous and 16-byte aligned, every
 *                     output is a dot product split in equal k-chunks; with
 *                     the matrix operand contiguous along the output instead
 *                     (16-byte aligned base and rows, any vector stride),
 *                     each workgroup wave accumulates a block of outputs over
 *                     a chunk of the k rows.  A few vectors (2 <= m <= 16, or
 *                     2 <= n <= 16 with m > 16; fp16/bf16 up to 8) against
 *                     k-contiguous rows, both operands k-contiguous and
 *                     16-byte aligned, are split the same way into blocks of
 *                     rows and k-chunks on MFMA.  Chunk sums are added in a
 *                     fixed order by a second kernel, so results are
 *                     reproducible.  Chosen explicitly, it returns
 *                     SK_ERR_UNSUPPORTED for other shapes or alignments, and
 *                     with ABFT.
 *  SK_SCHED_AUTO      SK_SCHED_GEMV_SPLIT for the shapes it takes (above)
 *                     (with default tile, grid and ABFT options); otherwise
 *                     SK_SCHED_XCD_ALIGNED with the tile instance, quantum and
 *                     grid chosen by the runtime model, or its data-parallel
 *                     form when the model predicts the split does not pay. */
typedef enum {
  SK_SCHED_AUTO = 0,
  SK_SCHED_DP = 1,
  SK_SCHED_SK_BASIC = 2,
  SK_SCHED_SK_HYBRID2 = 3,
  SK_SCHED_SK_HYBRID1 = 4,
  SK_SCHED_XCD_ALIGNED = 5,
  SK_SCHED_GEMV_SPLIT = 6
} sk_schedule;

/* One GEMM. */
typedef struct {
  int64_t m, n, k;
  float alpha;
  const void *A;
  int64_t lda;
  const void *B;
  int64_t ldb;
  float beta;
  void *C;
  int64_t ldc;
  sk_dtype dtype;
  sk_layout layout;
} sk_gemm_desc;

/* A fault to inject in ABFT mode (testing only).  The fault is applied to the
 * fp32 accumulator of element (row, col) of C in the work segment whose
 * k-iteration range (within the element's output tile) contains `iter`,
 * just before that segment is verified.  kind 0: add `value`; kind 1: flip
 * bit `bit` (0..31) of the fp32 accumulator. */
typedef struct {
  int64_t row, col;
  int32_t iter;
  int32_t kind;
  int32_t bit;
  float value;
} sk_fault;

#define SK_ABFT_MAX_RECORDS 64

/* One corrected (or uncorrectable) element found by ABFT. */
typedef struct {
  int64_t row, col;  /* element of C; -1 when not locatable */
  float delta;       /* faulty value minus corrected value */
  int32_t status;    /* 1 corrected, 2 uncorrectable (mismatch not located to one element) */
  int32_t tile;      /* output tile */
  int32_t seg_begin; /* first k-iteration of the verified segment */
} sk_abft_record;

/* ABFT report, written on the device (caller-owned device memory; the
 * library zeroes it at the start of each sk_gemm_ex call that passes it). */
typedef struct {
  int32_t detected;      /* verification domains with any mismatch */
  int32_t corrected;     /* elements corrected */
  int32_t uncorrectable; /* domains whose mismatch could not be located */
  int32_t n_records;     /* records produced; the first SK_ABFT_MAX_RECORDS are stored */
  sk_abft_record records[SK_ABFT_MAX_RECORDS];
  float max_ratio;       /* largest |checksum residual| / threshold over every row and column
                          * checked (a fault-free margin: below 1 nothing is flagged) */
  int32_t checked;       /* rows and columns checked */
} sk_abft_report;

/* Tile instances.  fp16/bf16 -- LARGE: 256 x 256 x 64 tiles, one
 * 512-thread workgroup per CU.  SMALL: 128 x 128 x 64 tiles, two 256-thread
 * workgroups per CU, for GEMMs with few large tiles (the page's observation
 * that a large tile loses on small, bandwidth-bound shapes, evaluation
 * section).  NARROW: for m <= 256 (SK_ERR_UNSUPPORTED above), BM x 256 x 64
 * tiles with BM = 64, 128, 192 or 256, the smallest that holds m, so that B
 * is read once; B streams into registers three iterations ahead
 * (memory-bound shapes with long k, the page's evaluation section).  AUTO
 * picks LARGE or SMALL by the runtime model.
 * fp32 -- LARGE: 128 x 128 x 32 tiles, two 256-thread workgroups per CU.
 * SMALL: 64 x 64 x 32 tiles, four 256-thread workgroups per CU (1024^3 is
 * one such tile per CU, with no partial exchange); not with ABFT
 * (SK_ERR_UNSUPPORTED), which runs on LARGE.  NARROW: SK_ERR_UNSUPPORTED.
 * AUTO picks LARGE or SMALL by the runtime model (LARGE with ABFT). */
typedef enum { SK_TILE_AUTO = 0, SK_TILE_LARGE = 1, SK_TILE_SMALL = 2, SK_TILE_NARROW = 3 } sk_tile;

/* Options for sk_gemm_ex.  Zero-initialised options mean: AUTO schedule, no
 * forced grid, ABFT off, default model constants, AUTO tile instance. */
typedef struct {
  int32_t schedule;         /* sk_schedule */
  int32_t forced_grid;      /* > 0: basic Stream-K with exactly this many workgroups (on the
                             * large tile unless `tile` names one) */
  int32_t abft;             /* nonzero: ABFT mode (checksums, verify, correct); SK_F32 only */
  int32_t hybrid_min_waves; /* full waves needed before the two-tile hybrid is used (default 1) */
  const sk_fault *faults;   /* device array of injected faults (testing), or NULL */
  int32_t n_faults;
  float abft_tau;           /* detection threshold factor c_tau (default 1) */
  /* grid-size model constants in units of one MAC iteration (0 = default):
   * fixed cost a, partial-output cost b, per-iteration cost c, per-peer cost d */
  float model_a, model_b, model_c, model_d;
  int32_t spin_limit_us;    /* fixup wait time-out in microseconds (0 = 2 s) */
  int32_t tile;             /* sk_tile: tile instance */
  int32_t test_flags;       /* testing only (0 otherwise): SK_TEST_NO_SIGNAL */
} sk_options;

/* test_flags bit: workgroups store their partial tiles but never signal
 * them, so every fixup wait of the call gives up after spin_limit_us (the
 * result is then wrong and the time-out is reported); forces the error path
 * of the bounded wait from the host.  Kernels always exit normally. */
#define SK_TEST_NO_SIGNAL 1

/* Plan of one call, for inspection (host only, needs no GPU when
 * sk_plan_query is given an explicit slot count).  For SK_SCHED_GEMV_SPLIT:
 * tiles = the number of outputs, tile_k = the k-chunk length in elements,
 * sk_blocks = chunks per output, iters_per_tile = 1; tile_m = tile_n = 0
 * for the dot-product form; tile_m = 0 and tile_n = the outputs one task
 * covers (64 x the elements in 16 bytes) for the form with the matrix
 * contiguous along the output; tile_m = the vectors and tile_n = the rows
 * one task covers for a few vectors; total_iters = the tasks (outputs or
 * output blocks times chunks), grid = workgroups of 256 threads; the other
 * fields that describe GEMM tiles are 0, and sk_plan_segments lists no
 * segments. */
typedef struct {
  int32_t tile_m, tile_n, tile_k; /* BLK_M, BLK_N, BLK_K of the kernel */
  int32_t slots;                  /* p: workgroups resident at once */
  int32_t grid;                   /* g: workgroups launched */
  int32_t schedule;               /* resolved sk_schedule (never AUTO) */
  int64_t tiles_m, tiles_n, tiles;/* t = tiles_m * tiles_n */
  int64_t iters_per_tile;         /* ceil(k / BLK_K) */
  int64_t total_iters;            /* t * iters_per_tile */
  int64_t sk_tiles;               /* tiles [0, sk_tiles) form the Stream-K region */
  int64_t sk_iters_q;             /* floor(sk_tiles * ipt / grid) (XCD_ALIGNED: floor(s * ipt / D)) */
  int64_t sk_iters_r;             /* (sk_tiles * ipt) mod grid: the first r workgroups take one more */
  int64_t dp_tiles;               /* tiles after the Stream-K region, dealt round-robin */
  int32_t full_waves;             /* w = floor(t / slots) */
  int32_t tail_tiles;             /* r = t mod slots */
  int32_t max_peers;              /* most partials any owner adds */
  int32_t packs;                  /* bit 0: A is repacked, bit 1: B is repacked */
  /* SK_SCHED_XCD_ALIGNED only (else 0): workgroup x covers region iterations
   * [floor(x*sk_blocks*ipt/phase_div), floor((x+1)*sk_blocks*ipt/phase_div));
   * tiles are ordered in bands of group_rows tile rows */
  int32_t phase_div;              /* D: quanta per tile (a multiple of 8) */
  int32_t sk_blocks;              /* s: quanta per workgroup */
  int32_t group_rows;             /* G */
  /* 1: the partials of a tile split over workgroups owner .. owner+P-1 are
   * combined in a binary tree: with r = x - owner, at level l = 0, 1, ... a
   * workgroup with bit l of r set stores the sum of its subtree and stops,
   * otherwise it adds the subtree of r + 2^l (if r + 2^l < P); the owner
   * (r = 0) writes the tile.  0: the owner adds the P-1 partials in order. */
  int32_t fixup_tree;
} sk_plan;

/* One work segment of a workgroup. */
typedef struct {
  int64_t tile;                 /* linear tile index: tile row * tiles_n + tile column */
  int64_t iter_begin, iter_end; /* k-iterations within the tile, [begin, end) */
  int32_t started;              /* holds iteration 0: the workgroup writes the tile */
  int32_t ended;                /* holds the tile's last iteration */
  int64_t last_peer;            /* owner that did not end the tile: highest peer it sums; else -1 */
} sk_segment;

/* C = alpha*A*B + beta*C with the AUTO schedule.  m == 0 or n == 0 returns
 * SK_OK without launching anything; k == 0 or alpha == 0 scales C by beta
 * (beta == 0 writes zeros without reading C). */
int sk_gemm(int64_t m, int64_t n, int64_t k, float alpha, const void *A, int64_t lda,
            const void *B, int64_t ldb, float beta, void *C, int64_t ldc, sk_dtype dtype,
            sk_layout layout, hipStream_t stream);

/* Same as sk_gemm with options.  `opts` may be NULL.  `report` is a device
 * pointer to an sk_abft_report (required when opts->abft is set, else
 * ignored).  The kernels walk a schedule in 32-bit integers: a schedule
 * chosen explicitly whose positions or quanta products would reach 2^31
 * (k of several million with the XCD-aware schedule) returns
 * SK_ERR_UNSUPPORTED; AUTO then takes the two-tile hybrid, else the
 * data-parallel order.  The k-contiguous copy of an operand the kernels
 * cannot read in place (plan packs bits; rows * ceil(k/64) * 64 elements per
 * copy) is kept in the stream's workspace, one buffer for A and one for B
 * (grown when a call needs more, after synchronising the stream; freed by
 * sk_release_workspace; SK_ERR_NO_MEMORY when it cannot be had).  In ABFT
 * mode the operands' checksum encodings and
 * detection-threshold inputs, at most about 4 * ((tiles_m + tiles_n) * 32 *
 * ceil(k/32) + (m + n) * (ceil(k/64) + 1)) bytes for 128 x 128 tiles (at
 * least 4 MiB), and one 32-bit counter per tile of A and B, are kept in the
 * stream's workspace (grown when a call needs more, after synchronising the
 * stream; freed by sk_release_workspace). */
int sk_gemm_ex(const sk_gemm_desc *desc, const sk_options *opts, sk_abft_report *report,
               hipStream_t stream);

/* Bytes of partial-tile scratch the allocation-free entry point holds per
 * GPU (256 partial tiles of 256 x 256 fp32). */
#define SK_NOALLOC_PARTIAL_BYTES (64u * 1024u * 1024u)

/* Allocation-free form of sk_gemm_ex, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  Same GEMM, plans and kernels as
 * sk_gemm_ex, but it calls no allocating routine: the partial tiles, flags
 * and status word of the cross-workgroup fixup live in a static device array
 * of the library (SK_NOALLOC_PARTIAL_BYTES plus 128 KiB; each GPU the
 * library runs on holds its own copy until the process ends).  The first
 * call on a device looks the array up and clears its flags with a fill
 * kernel on `stream`.  Every call on one GPU shares that array and leaves it
 * as the call ended: calls that overlap on one GPU (other streams, other
 * host threads) race and must not be issued.  Refused: ABFT mode and
 * operands that would need a repacked copy (SK_ERR_UNSUPPORTED; the
 * conditions for reading an operand in place are listed with sk_layout:
 * plan packs bits 0), and plans needing more than 16384
 * workgroups or more partial-tile bytes than SK_NOALLOC_PARTIAL_BYTES
 * (SK_ERR_TOO_LARGE: a forced grid above the slot count on the large
 * fp16/bf16 tile, or a matrix-vector split with more chunk sums).  Time-outs
 * of the fixup wait are reported by sk_device_status() as for sk_gemm_ex. */
int sk_gemm_noalloc(const sk_gemm_desc *desc, const sk_options *opts, hipStream_t stream);

/* Plan the call would use.  slots > 0 plans for that many resident
 * workgroups of the large-tile kernel (the small-tile instance runs two
 * workgroups where the large one runs one, so it is planned for 2 * slots)
 * without touching the GPU; slots == 0 asks the current device. */
int sk_plan_query(const sk_gemm_desc *desc, const sk_options *opts, int32_t slots, sk_plan *out);

/* Segments of workgroup `wg` under `plan`, in execution order.  Writes at
 * most `cap` entries and returns the number of segments (which may exceed
 * cap), or a negative sk_status. */
int64_t sk_plan_segments(const sk_plan *plan, int64_t wg, sk_segment *out, int64_t cap);

/* Error words of the current device's workspaces and of the allocation-free
 * entry point's scratch: SK_OK or SK_ERR_FIXUP_TIMEOUT (a time-out not yet
 * reported by a later call); synchronises the device and clears them. */
int sk_device_status(void);

/* Text of a status code, and of the last HIP error seen by the library. */
const char *sk_strerror(int status);
const char *sk_last_hip_error(void);

/* Frees every workspace of the calling process (synchronises the device). */
int sk_release_workspace(void);

/* Library version string. */
const char *sk_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SK_GEMM_H */
