/*
 * q8gemv.h -- C ABI of the MI355X (gfx950) Q8_0 decode matvec library.
 *
 * The operation (page "IV.4: One command buffer per token", section "Eight
 * kernels", the q8_matvec kernel and the paragraph after it):
 *
 *   W is a p x n matrix in Q8_0: p rows, each of n/32 consecutive 34-byte
 *   blocks; a block is a little-endian IEEE binary16 scale d followed by 32
 *   two's-complement int8 quants q_0..q_31.  For every row r
 *
 *       y[r] = sum_b d(r,b) * sum_{j<32} q(r,b,j) * x[32b + j]
 *
 *   with x and y float32.  The result overwrites y (no accumulate).
 *
 * Conventions for every entry point:
 *   - All data pointers (x, w, y, X, Y) are DEVICE pointers owned by the
 *     caller; the library never frees or retains them except as stated for
 *     chains.  `stream` is a hipStream_t passed as void* (NULL = the legacy
 *     default stream).
 *   - Arguments are validated before anything is enqueued; a failed
 *     validation enqueues nothing and returns a negative q8_status.  The
 *     calls never fall back to another implementation.
 *   - Calls are asynchronous: they enqueue on `stream` and return.  Only
 *     q8_0_decode_chain in Q8_MODE_SYNC_EACH and q8_0_stream_wait block.
 *   - Alignment: w and x (X) must be 16-byte aligned; y (Y) 4-byte aligned.
 *     (Rows of X are n floats apart, n a multiple of 32, so every row of an
 *     aligned X is aligned too.)
 *   - y (Y) must not overlap x (X) or w.
 *   - Sizes: n is a positive multiple of 32 and at most Q8_MAX_N; p is
 *     positive and at most Q8_MAX_P; small-batch m is in 1..Q8_MAX_M.
 *   - No entry point allocates, frees or synchronizes device memory on its
 *     own except q8_0_chain_create/destroy (and, in q8step.h, the step's
 *     create/destroy), which own what they allocate.  Calls whose kernels
 *     need scratch memory (the small-batch product; in q8step.h the
 *     standalone attention and argmax) take a caller-owned device workspace
 *     whose size a host-only query returns; it is 256-byte aligned, may hold
 *     anything beforehand (the small-batch arrival counters carry a per-call
 *     tag; attention and argmax clear theirs), and must not be used by two
 *     calls that may overlap.
 *   - Results are bitwise reproducible run to run for the same inputs,
 *     shapes and device: every sum runs in a fixed order (the small-batch
 *     product counts arrivals with an atomic counter, but adds partial sums
 *     in a fixed order).  For m = 1 the order depends on n only: every
 *     launch shape, chain mode and chain flag gives the same bits as
 *     q8_0_gemv for the same x and w.
 *   - Accuracy: |y - exact| <= 1e-5 * sum_j |w_j x_j| + 1e-6 per output for
 *     finite inputs (float32 arithmetic with a bounded summation depth).
 */
#ifndef Q8GEMV_H
#define Q8GEMV_H

#include <stddef.h>
#include <stdint.h>

/* Only the entry points below are exported from libq8gemv.so. */
#ifndef Q8_API
#define Q8_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum q8_status {
    Q8_OK = 0,
    Q8_ERR_INVALID_ARG = -1, /* null pointer, unknown mode or flag, bad handle */
    Q8_ERR_SHAPE = -2,       /* n, p or m out of range (zero is out of range) */
    Q8_ERR_ALIGN = -3,       /* a pointer is not aligned as required */
    Q8_ERR_ALIAS = -4,       /* an output overlaps an input */
    Q8_ERR_NO_DEVICE = -5,   /* no HIP device is visible */
    Q8_ERR_HIP = -6,         /* the HIP runtime reported an error (see q8_0_last_error) */
    Q8_ERR_TIMEOUT = -7,     /* q8_0_stream_wait ran out of time */
    Q8_ERR_UNSUPPORTED = -8  /* the current device is not gfx950 */
};

#define Q8_BLOCK_QUANTS 32
#define Q8_BLOCK_BYTES 34
#define Q8_MAX_N (1 << 20)         /* columns */
#define Q8_MAX_P 0x7fffffff        /* rows */
#define Q8_MAX_M 16                /* small-batch rows of X */
#define Q8_MAX_CHAIN_OPS 65535

/*
 * y = W x for one p x n Q8_0 matrix.
 * Argument order follows the page's kernel: (x, w, out, n, p) -- section
 * "Eight kernels", q8_matvec, buffers 0..4.
 *   x : float32[n], device, 16-B aligned.   w : p * (n/32) * 34 bytes, device, 16-B aligned.
 *   y : float32[p], device, written.
 */
Q8_API int q8_0_gemv(const float *x, const void *w, float *y, int64_t n, int64_t p,
              void *stream);

/*
 * q8_0_gemv on an explicit launch shape, for n a multiple of 256 (else
 * Q8_ERR_SHAPE): lanes_per_row (1, 2 or 4) lanes share each row, so a wave
 * covers 64 / lanes_per_row rows; `waves` (1, 2 or 4) waves per workgroup
 * split each row's groups; each wave stages its weights in `stages` (1 or 2)
 * LDS buffers of 17 KiB.  Shapes whose workgroup would need more than
 * 160 KiB of LDS are refused (Q8_ERR_INVALID_ARG).  The result is bitwise
 * identical to q8_0_gemv's for every shape; the shape only changes the
 * launch (for measurements and for tests of that identity).  Allocates
 * nothing.
 */
Q8_API int q8_0_gemv_shaped(const float *x, const void *w, float *y, int64_t n, int64_t p,
                            int lanes_per_row, int waves, int stages, void *stream);

/*
 * Y = X W^T for m in 1..16 activation rows in one pass over W: the small-batch
 * matvec of multi-sequence decode (page "Metal Backend Optimizations",
 * section 0.3, the batched-matvec kernel family left open for 2..8 tokens;
 * page "minfer Metal Backend Design", section 4.4, the matmul tiers).
 *   X : float32[m][n] row-major, device.   Y : float32[m][p] row-major, device.
 * Each Y[i] equals what q8_0_gemv gives for x = X[i] to the same accuracy.
 * workspace: a device buffer of at least the bytes q8_0_gemm_smallm_workspace
 * gives for (m, n, p, Q8_SMALLM_AUTO) on the current device (0 for m = 1:
 * then it may be NULL); 256-byte aligned, not overlapping X, w or Y
 * (Q8_ERR_ALIGN, Q8_ERR_INVALID_ARG if too small, Q8_ERR_ALIAS).  Its
 * contents before the call do not matter; calls that may run at the same
 * time need workspaces of their own.
 */
Q8_API int q8_0_gemm_smallm(const float *X, const void *w, float *Y, int64_t m,
                     int64_t n, int64_t p, void *workspace, size_t workspace_bytes, void *stream);

/*
 * *bytes = the workspace q8_0_gemm_smallm(_kernel) needs for (m, n, p) with
 * `kernel` on the current device (its CU count sets the split of the work).
 * Enqueues nothing.  Q8_ERR_SHAPE if the kernel does not take the shape.
 */
Q8_API int q8_0_gemm_smallm_workspace(int64_t m, int64_t n, int64_t p, int kernel, size_t *bytes);

/*
 * q8_0_gemm_smallm for callers that cannot allocate or pass device memory of
 * their own (code under stream capture, tight serving loops, harnesses that
 * forbid allocation): the same kernels and the same results, with the
 * workspace taken from a scratch array inside the library, 32 MiB on each
 * GPU it runs on, held until the process ends.  Allocates nothing.  One
 * exception to "the same kernels": where q8_0_gemm_smallm would run
 * Q8_SMALLM_KS with more than 16 MiB of per-range sums (rows of whole
 * groups, m and n large, e.g. m = 16, n = 3584, p = 152064), this call runs
 * Q8_SMALLM_MFMA instead, which needs far less; its results then meet the
 * same bar but round differently.
 * Q8_ERR_SHAPE (with the bytes needed in q8_0_last_error) when the call needs
 * more than that (q8_0_gemm_smallm_workspace tells).  Every call on one GPU
 * shares its array: calls that may overlap on one GPU (other streams,
 * other threads) race and must not be issued.
 */
Q8_API int q8_0_gemm_smallm_noalloc(const float *X, const void *w, float *Y, int64_t m,
                                    int64_t n, int64_t p, void *stream);

/* Small-batch kernels (q8_0_gemm_smallm_kernel). */
#define Q8_SMALLM_AUTO 0  /* the choice q8_0_gemm_smallm makes */
#define Q8_SMALLM_VALU 1  /* vector units, a lane per row, up to 4 rows of X per pass over W */
#define Q8_SMALLM_MFMA 2  /* bf16 matrix cores on X split exactly in three parts; n % 128 == 0 */
#define Q8_SMALLM_VROW 3  /* vector units, lanes over a row and a block pair, two waves per
                             workgroup; n % 256 == 0 and m <= 3 */
#define Q8_SMALLM_VROW1 4 /* the same with one wave per workgroup */
#define Q8_SMALLM_KS 5    /* bf16 matrix cores on X split exactly in three parts, each column
                             range's parts held in LDS by the workgroups that stream its rows;
                             n % 256 == 0 */

/*
 * *kernel = the kernel (Q8_SMALLM_*, never AUTO) q8_0_gemm_smallm runs for
 * (m, n, p), m = 2..16, on the current device.  Enqueues nothing.
 * Q8_ERR_SHAPE for a shape out of range, Q8_ERR_INVALID_ARG for a null
 * kernel, Q8_ERR_NO_DEVICE without a device.
 */
Q8_API int q8_0_gemm_smallm_choice(int64_t m, int64_t n, int64_t p, int *kernel);

/*
 * q8_0_gemm_smallm on a named kernel (for measurements and for tests of each
 * kernel); Q8_ERR_SHAPE if that kernel does not take (m, n).  Each kernel
 * meets the same accuracy bar; their roundings differ.
 */
Q8_API int q8_0_gemm_smallm_kernel(const float *X, const void *w, float *Y, int64_t m,
                                   int64_t n, int64_t p, int kernel, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * One decode step's chain of matvecs, recorded once and replayed per token
 * (page "IV.4: One command buffer per token", section "One command buffer":
 * all of a step's dispatches are encoded once, committed and waited on once).
 */
typedef struct q8_0_op {
    const float *x;  /* float32[n], 16-B aligned */
    const void *w;   /* Q8_0, p rows of n/32 blocks, 16-B aligned */
    float *y;        /* float32[p] */
    int64_t n;
    int64_t p;
} q8_0_op;

typedef struct q8_0_chain q8_0_chain; /* opaque */

/* chain_create flags (may be combined) */
#define Q8_CHAIN_FUSE 0u    /* merge runs of mutually independent ops into one launch */
#define Q8_CHAIN_PER_OP 1u  /* one kernel launch per op, in array order */
#define Q8_CHAIN_SPLIT_K 2u /* for ops that wait on each other (a real decode step): plan
                               every launch for latency -- short row tiles, each row's groups
                               split over the waves of a workgroup -- rather than for the
                               steady state of a long launch; the same bits either way */
#define Q8_CHAIN_XQ 4u      /* every op as q8_0_gemv_q8q8: x quantized to Q8_0, integer dots */

/* decode_chain modes */
#define Q8_MODE_GRAPH 0     /* replay the recorded hipGraph: one host call per token (a chain
                               of one launch issues that launch directly) */
#define Q8_MODE_EAGER 1     /* re-issue the chain's launches on the stream */
#define Q8_MODE_SYNC_EACH 2 /* one launch, then wait for it, per launch */

/*
 * Validate the ops (each as q8_0_gemv would), plan the launches and record
 * them into a hipGraph on the current device.  Ops run in array order: an op
 * that reads (x) or writes (y) memory that an earlier op writes, or writes
 * memory an earlier op reads, starts only after that earlier op has finished;
 * with Q8_CHAIN_FUSE, maximal runs of ops with no such overlap share one
 * launch.  The pointers in `ops` are baked into the recording: they must stay
 * valid, at the same addresses, until q8_0_chain_destroy.  The handle owns a
 * small device table (op descriptors and the tile schedule), a private
 * capture stream and the graph; a token's replay allocates nothing.  Every
 * op's outputs are bitwise those of q8_0_gemv (q8_0_gemv_q8q8 with
 * Q8_CHAIN_XQ), whatever the flags and mode.  Replays of one chain must not
 * overlap in time (they share their outputs).
 * On failure *out is set to NULL and nothing is leaked.
 */
Q8_API int q8_0_chain_create(const q8_0_op *ops, int64_t n_ops, uint32_t flags,
                      q8_0_chain **out);

/*
 * The integer path (page "IV.4: One command buffer per token", section
 * "Eight kernels": the CPU kernel beside q8_matvec quantizes the activations
 * and multiplies integers; page "minfer Metal Backend Design", ADR-0013).
 * x is quantized to Q8_0 blocks -- per 32 values d = amax/127 (float32),
 * code = x/d rounded half away from zero (0 when d == 0), d stored as
 * binary16 (nearest, ties to even); the pages do not print this rule, it is
 * the reading taken -- and each block's dot is an integer sum:
 *   y[r] = sum_b d_w(r,b) * d_x(b) * sum_j q_w(r,b,j) * q_x(b,j).
 * Arguments, validation and errors as q8_0_gemv; x must be finite.  The codes
 * are bit-identical to q8_0_quantize's; y is held to the same bar as
 * q8_0_gemv, against that integer definition.  Allocates nothing.
 */
Q8_API int q8_0_gemv_q8q8(const float *x, const void *w, float *y, int64_t n, int64_t p,
                   void *stream);

/*
 * x (n floats, n a positive multiple of 32, at most 2^31, 4-byte aligned) ->
 * n/32 Q8_0 blocks of 34 bytes at xq (the weight layout; no alignment
 * needed; must not overlap x), by the rule above.  Exact: the bytes are
 * decided by float32 operations.
 */
Q8_API int q8_0_quantize(const float *x, void *xq, int64_t n, void *stream);

/* Run one token's chain on `stream` in the given mode. */
Q8_API int q8_0_decode_chain(q8_0_chain *chain, int mode, void *stream);

/*
 * Launch plans, host only (nothing is enqueued, no device is needed): how
 * q8_0_gemv and q8_0_chain_create would launch on a GPU of `cus` compute
 * units (256 on MI355X).  For inspection and for tests of the planners.
 *
 * q8_0_gemv_plan: rows of whole 272-byte groups (n % 256 == 0) run on the
 * rows-and-group-slots kernel with `lanes_per_row` (1, 2, 4) lanes per row,
 * `waves` (1, 2, 4) waves sharing a tile's rows and `stages` (1, 2) weight
 * stages, one workgroup per tile of `tile_rows` rows (at most
 * 64 / lanes_per_row: fewer where that spreads the tiles evenly over the
 * CUs); other widths on the super-row kernel (lanes_per_row = stages =
 * tile_rows = 0, `waves` per workgroup).
 */
Q8_API int q8_0_gemv_plan(int64_t n, int64_t p, int64_t cus, int *lanes_per_row, int *waves,
                          int *stages, int *tile_rows, int64_t *workgroups);

#define Q8_LAUNCH_ROWS 0         /* one op, rows-and-group-slots kernel (its latency plan) */
#define Q8_LAUNCH_SUPERROWS 1    /* one op of another width, super-row kernel */
#define Q8_LAUNCH_FUSED 2        /* independent ops of whole-group rows in one launch */
#define Q8_LAUNCH_FUSED_MIXED 3  /* independent ops of mixed widths in one launch */

/* One launch of a chain's token. */
typedef struct q8_0_launch_plan {
    int32_t kind;           /* Q8_LAUNCH_* */
    int32_t lanes_per_row;  /* as q8_0_gemv_plan (0: super-row kernel) */
    int32_t waves;
    int32_t stages;
    int32_t tile_rows;      /* rows per tile: as q8_0_gemv_plan for one-op launches, 64 / lanes_per_row
                               for fused ones (mixed: 64 rows or one super-row tile); 0 for the
                               super-row kernel */
    int32_t pad_;
    int64_t first_op;       /* the launch computes ops[first_op .. first_op + n_ops) */
    int64_t n_ops;
    int64_t workgroups;
    int64_t first_tile;     /* fused launches: workgroup g does item first_tile + g of the
                               tile lists; -1 for one-op launches */
} q8_0_launch_plan;

/*
 * q8_0_chain_plan: the launches q8_0_chain_create(ops, n_ops, flags) would
 * record, in order, and for fused launches the item of every workgroup:
 * tile_op[k] = the op (index into ops), tile_id[k] = the tile within it (of
 * tile_rows rows; in mixed launches bit 31 marks a tail tile, rows past the
 * op's super-rows).  The same validation as q8_0_chain_create (the
 * pointers are compared, never dereferenced).  *n_launches and *n_tiles are
 * always set; the arrays are filled only when they are given and hold that
 * many entries.
 */
Q8_API int q8_0_chain_plan(const q8_0_op *ops, int64_t n_ops, uint32_t flags, int64_t cus,
                           q8_0_launch_plan *launches, int64_t max_launches, int64_t *n_launches,
                           int64_t *tile_op, uint32_t *tile_id, int64_t max_tiles, int64_t *n_tiles);

/* Kernel launches one token costs (1 .. n_ops); negative status on a bad handle. */
Q8_API int q8_0_chain_launches(const q8_0_chain *chain);

/* Release the handle (NULL is accepted).  The caller must make sure no
 * replay is still running. */
Q8_API int q8_0_chain_destroy(q8_0_chain *chain);

/*
 * Wait until all work on `stream` has finished, for at most timeout_ms
 * milliseconds (timeout_ms < 0: no limit).  Returns Q8_ERR_TIMEOUT when the
 * time runs out; the work itself is not cancelled.  A bounded wait with a
 * status check follows page "minfer Metal Backend Design", section 4.8.
 */
Q8_API int q8_0_stream_wait(void *stream, int64_t timeout_ms);

/* Static description of a status code. */
Q8_API const char *q8_0_status_string(int status);

/* Detail of the last error raised on the calling thread ("" if none). */
Q8_API const char *q8_0_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* Q8GEMV_H */
