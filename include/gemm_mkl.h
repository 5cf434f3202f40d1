/*
 * gemm_mkl.h -- C ABI of the MI355X (gfx950) tiled dense GEMM library.
 *
 * Operation (for every l < L, m < M, n < N):
 *
 *     C[l][m][n] = epilogue( sum_{k<K} A[l][m][k] * B[l][n][k] )
 *
 * The operand modes are those of the persistent dense GEMM kernel on
 * "深入解析 CUTLASS CuTe DSL 的 JIT 函数参数生成机制" (section 2.3): A has modes
 * (M,K,L), B has (N,K,L), C has (M,N,L).  The epilogue is an elementwise
 * function chosen at compile time (same page, section 2.3, and the compile-time
 * ReLU of section 7 of "CUTLASS CuTe DSL 控制流编程指南"); SiLU is the third.
 *
 * Layout: packed, batch outermost, K contiguous.
 *     A: L*M*K elements, element (l,m,k) at ((l*M + m)*K + k)
 *     B: L*N*K elements, element (l,n,k) at ((l*N + n)*K + k)
 *     C: L*M*N elements, element (l,m,n) at ((l*M + m)*N + n)
 * One dtype covers A, B and C; products are formed in the operand precision
 * and summed in fp32; the epilogue runs on the fp32 sum, which is then rounded
 * to the output dtype (round to nearest even).
 *
 * Pointers: A, B, C are DEVICE pointers owned by the caller; the library never
 * allocates, frees or retains them.  C must share no byte with A or B (a C
 * that does is INVALID_VALUE, checked on the addresses before any launch; A
 * and B may overlap each other, both are only read).  Each base
 * pointer must be aligned to its element size.  The tile kernels read A and B
 * in 16-byte pieces: when K*sizeof(element) is not a multiple of 16, or A or
 * B is not 16-byte aligned, the call first copies the operand(s) into rows of
 * Kp elements (K rounded up to 16 bytes, zero-filled past K) in the workspace
 * and runs the tile kernels on those (plan.packed = 1; the zeros add nothing,
 * so the result is that of the tile kernels at the padded K).  A C that is
 * not aligned to 4 elements, or GEMM_MKL_OPT_FORCE_GENERAL, takes a slower
 * general kernel instead (same results up to fp32 summation order).
 *
 * Stream: `stream` is a hipStream_t (NULL = the default stream).  Calls only
 * enqueue work and return without synchronising; a kernel fault surfaces at
 * the caller's next synchronisation.  Calls on different streams may run
 * concurrently; two calls that share an internal split-K workspace are
 * serialised by the stream they were issued on (the workspace is per device
 * and per stream).
 *
 * Errors: every argument check happens before any HIP call, so a rejected call
 * touches no device state and leaves C unchanged.  The return value is one of
 * the GEMM_MKL_STATUS_* codes below.
 */
#ifndef GEMM_MKL_H_
#define GEMM_MKL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Operand / output dtype (A, B and C share it; accumulation is always fp32). */
enum {
    GEMM_MKL_F32 = 0,
    GEMM_MKL_F16 = 1,
    GEMM_MKL_BF16 = 2
};

/* Epilogue applied to the fp32 accumulator before the output conversion. */
enum {
    GEMM_MKL_EPI_IDENTITY = 0, /* y = x                                  */
    GEMM_MKL_EPI_RELU = 1,     /* y = x > 0 ? x : 0  (so -0 becomes +0)   */
    GEMM_MKL_EPI_SILU = 2      /* y = x * sigmoid(x) = x / (1 + exp(-x)) */
};

/* Status codes. */
enum {
    GEMM_MKL_STATUS_OK = 0,
    GEMM_MKL_STATUS_INVALID_VALUE = -1,        /* null pointer for a non-empty problem,
                                                  negative size, size overflow,
                                                  pointer not aligned to its element,
                                                  an output sharing bytes with an
                                                  input or the workspace,
                                                  prefetch_stages < -1, bad option */
    GEMM_MKL_STATUS_UNSUPPORTED_DTYPE = -2,    /* dtype not one of GEMM_MKL_F32/F16/BF16 */
    GEMM_MKL_STATUS_UNSUPPORTED_EPILOGUE = -3, /* epilogue not one of GEMM_MKL_EPI_* */
    GEMM_MKL_STATUS_WORKSPACE = -4,            /* caller workspace too small, or the
                                                  internal one could not be allocated */
    GEMM_MKL_STATUS_HIP_ERROR = -5,            /* a HIP runtime call failed */
    GEMM_MKL_STATUS_NOT_AVAILABLE = -6         /* the forced kernel configuration /
                                                  prefetch depth does not exist or does
                                                  not fit this problem */
};

/*
 * The GEMM.  Sizes are element counts (M, N, K, L >= 0).
 *   M*N*L == 0  -> success, nothing launched.
 *   K == 0      -> C = epilogue(0) = 0.
 * The library picks the kernel configuration (tile, prefetch depth, split-K
 * factor) from the problem shape.  When it splits K, it sums the fp32 partial
 * results in a fixed order in a workspace it owns (see gemm_mkl_release_workspace);
 * results are bitwise reproducible from run to run.
 */
int gemm_mkl(const void *A, const void *B, void *C,
             int64_t M, int64_t N, int64_t K, int64_t L,
             int dtype, int epilogue, void *stream);

/*
 * Options for gemm_mkl_ex.  Initialise with gemm_mkl_opts_init (all automatic),
 * then set what you need.
 *
 * prefetch_stages: number of K chunks loaded ahead of the one being consumed
 *   (the global -> LDS prefetch ring holds prefetch_stages + 1 chunks); 0 is
 *   load-then-use with no prefetch, -1 is automatic.  This is the
 *   prefetch_stages of the software-pipelined loop in section 3 of
 *   "CUTLASS CuTe DSL 控制流编程指南": a prologue loads the first stages, then
 *   iteration i loads stage i + prefetch_stages while it consumes stage i, and
 *   a negative depth is an error there as it is here.  Below -1 is
 *   INVALID_VALUE (the depth must be 0 or greater); a depth that no kernel
 *   configuration provides is NOT_AVAILABLE.
 * split_k: number of K ranges computed by separate workgroups and summed in
 *   ascending order of range (0 = auto, 1 = no split, at most 16).  Ranges
 *   that would be empty are dropped.  A value >= 1 also rules out the
 *   stream-K kernel unless GEMM_MKL_OPT_STREAMK is set (with split_k > 1 that
 *   combination is NOT_AVAILABLE).
 * config_id: index into the kernel configuration table (-1 = auto); see
 *   gemm_mkl_config_name.  A configuration of another dtype is NOT_AVAILABLE.
 * flags: GEMM_MKL_OPT_FORCE_GENERAL selects the general kernel;
 *   GEMM_MKL_OPT_STREAMK / GEMM_MKL_OPT_NO_STREAMK force / forbid the stream-K
 *   kernel (one workgroup per compute unit, each summing an equal share of all
 *   (tile, K-chunk) units; tiles cut between workgroups are summed in a fixed
 *   order, so results stay bitwise reproducible).  The automatic plan uses
 *   stream-K only when GEMM_MKL_STREAMK=-1 is set in the environment.
 *   GEMM_MKL_OPT_PERSISTENT / GEMM_MKL_OPT_NO_PERSISTENT force / forbid the
 *   persistent grid (one workgroup per compute unit, each taking every
 *   G-th tile and running one prefetch ring across its tiles, so a tile's
 *   first loads overlap the end of the tile before it).  It exists for the
 *   producer-wave configurations, without a K split; each tile is computed
 *   exactly as by the data-parallel grid (same chunk order), so results are
 *   bitwise equal to it.  The automatic plan does not use it (it measured no
 *   faster than the data-parallel grid); GEMM_MKL_PERSISTENT=-1 lets the plan
 *   take it whenever there are more tiles than compute units, =1 always.
 *   GEMM_MKL_OPT_FIXUP / GEMM_MKL_OPT_NO_FIXUP: a split plan sums its pieces
 *   inside the GEMM kernel (split_k 2..6): the S pieces of a tile run on one
 *   XCD, each stores its fp32 partial (it stays in that XCD's L2) and counts
 *   itself in the tile's counter word with one atomic, and the last piece
 *   adds the partials in ascending split order, applies the epilogue and
 *   stores C.  No workgroup waits for another.  Results equal the split-K
 *   grid with the separate reduction bit for bit.  GEMM_MKL_FIXUP=0/1/-1 in
 *   the environment: never / always / by the model (the default, -1).
 * workspace / workspace_bytes: caller-owned device memory for split-K or
 *   stream-K partial sums and repacked operands (NULL = use the library's
 *   internal workspace).  It must hold the plan's workspace_bytes
 *   (gemm_mkl_get_plan, which assumes 16-byte aligned pointers: a misaligned
 *   A or B also needs its repacked copy, L * rows * Kp * element bytes
 *   rounded up to 256) and be 256-byte aligned, sharing no byte with A, B
 *   or C (INVALID_VALUE otherwise); too small is
 *   GEMM_MKL_STATUS_WORKSPACE, before anything is launched.  A stream-K or
 *   fix-up plan uses its first plan.counter_bytes bytes as per-tile counters:
 *   they must be zero before the first such call with that workspace, and
 *   every completed call leaves them zero.
 *
 * The environment variables GEMM_MKL_FORCE_CONFIG, GEMM_MKL_STAGES and
 * GEMM_MKL_SPLIT_K supply the same three choices when opts leaves them
 * automatic (for sweeps); GEMM_MKL_STREAMK=0/1/-1 never / always / by model
 * uses stream-K; GEMM_MKL_PERSISTENT=0/1/-1 never (default) / always / when
 * there are more tiles than compute units uses the persistent grid; GEMM_MKL_GROUP_M
 * sets the tile-raster group height (default 4; 6 inside the groups of
 * gemm_mkl_grouped);
 * GEMM_MKL_LOG=1 prints each call's plan to stderr;
 * GEMM_MKL_WORKSPACE_LIMIT=<bytes> caps the internal workspace.  They are
 * read once, at the first call.  Plans are cached per (sizes, dtype, pointer
 * alignment, options), so a repeated call does no planning work.
 */
typedef struct gemm_mkl_opts {
    int32_t prefetch_stages; /* -1 = auto */
    int32_t split_k;         /* 0 = auto */
    int32_t config_id;       /* -1 = auto */
    int32_t flags;           /* GEMM_MKL_OPT_* bits */
    void *workspace;         /* device pointer or NULL */
    size_t workspace_bytes;
} gemm_mkl_opts;

/* flags */
enum {
    GEMM_MKL_OPT_FORCE_GENERAL = 1, /* use the general (unaligned-capable) kernel */
    GEMM_MKL_OPT_STREAMK = 2,       /* use the stream-K kernel (NOT_AVAILABLE if no
                                       configuration of the dtype has one, or with
                                       split_k > 1) */
    GEMM_MKL_OPT_NO_STREAMK = 4,    /* never use the stream-K kernel */
    GEMM_MKL_OPT_PERSISTENT = 8,    /* use the persistent grid (NOT_AVAILABLE unless the
                                       chosen configuration has one, with split_k 1 and
                                       its own prefetch depth) */
    GEMM_MKL_OPT_NO_PERSISTENT = 16, /* never use the persistent grid */
    GEMM_MKL_OPT_FIXUP = 32,        /* split plans sum their pieces inside the GEMM kernel
                                       (the in-kernel fix-up; NOT_AVAILABLE with a forced
                                       split when the configuration has no fix-up kernel,
                                       split_k > 6 or a depth other than its own) */
    GEMM_MKL_OPT_NO_FIXUP = 64,     /* split plans use the separate reduction kernel */
    GEMM_MKL_OPT_FIXUP_RECOMPUTE = 128 /* test hook: the piece that finishes a fix-up tile
                                       computes every other piece's partial itself instead
                                       of reading it (the path taken when a partial was
                                       written on another XCD); same results */
};

/* Initialise opts to "all automatic". */
void gemm_mkl_opts_init(gemm_mkl_opts *opts);

/* The GEMM with explicit options (opts == NULL is the same as gemm_mkl). */
int gemm_mkl_ex(const void *A, const void *B, void *C,
                int64_t M, int64_t N, int64_t K, int64_t L,
                int dtype, int epilogue, void *stream,
                const gemm_mkl_opts *opts);

/*
 * gemm_mkl_ex for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * computes what gemm_mkl_ex computes (same plans, same kernels, same bits
 * for the same plan), but the split-K partial sums and repacked operands live
 * in a fixed device scratch array of GEMM_MKL_NOALLOC_SCRATCH_BYTES that the
 * library holds on each device it runs on (allocated with the library's code
 * when the library is first used on that device, and kept until the process
 * ends).  The call allocates and frees nothing.
 *
 * opts: as for gemm_mkl_ex, except that opts->workspace must be NULL and
 *   workspace_bytes 0 (INVALID_VALUE otherwise) and GEMM_MKL_OPT_STREAMK is
 *   NOT_AVAILABLE (stream-K is never used here).  The automatic plan only
 *   considers K splits whose partial sums fit the scratch; a plan that still
 *   needs more than GEMM_MKL_NOALLOC_SCRATCH_BYTES (a forced split, or
 *   repacked operands: K * element bytes not a multiple of 16, A or B not
 *   16-byte aligned) returns GEMM_MKL_STATUS_WORKSPACE before anything is
 *   launched, with C untouched.
 *
 * Every call on a device uses that device's one scratch array.  Calls that
 * may overlap on one device (concurrent streams, or calls from several
 * threads) race on it and are undefined; calls issued in order on one stream
 * are safe.  No part of the scratch has to start at zero.  Ownership of A, B
 * and C and the status codes are as for gemm_mkl_ex.
 */
#define GEMM_MKL_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

int gemm_mkl_noalloc(const void *A, const void *B, void *C,
                     int64_t M, int64_t N, int64_t K, int64_t L,
                     int dtype, int epilogue, void *stream,
                     const gemm_mkl_opts *opts);

/*
 * Grouped GEMM: G problems that share N and K but each have their own number
 * of rows, as the grouped matrix product reached through framework adapters on
 * "深入解析 CUTLASS CuTe DSL 的 JIT 函数参数生成机制" (section 5) does.  Group g
 * owns rows [offs[g - 1], offs[g]) of A and C (offs[-1] = 0) and its own B[g]:
 *
 *   C[r][n] = epilogue( sum_k A[r][k] * B[g][n][k] )   for r in group g
 *
 * A:    device pointer, [total_m][K], K contiguous.
 * B:    device pointer, [G][N][K], K contiguous.
 * C:    device pointer, [total_m][N], N contiguous; rows outside every group
 *       are left untouched.
 * offs: DEVICE pointer to G int32 cumulative row ends (offs[G - 1] normally
 *       equals total_m; empty groups repeat the previous end).  The kernels
 *       read it on the GPU, so the call needs no host synchronisation; they
 *       clamp it to a non-decreasing sequence in [0, total_m], so offsets
 *       outside that range never address rows outside A or C.
 * dtype, epilogue, stream: as for gemm_mkl; accumulation is fp32.
 * opts: NULL for automatic; config_id and prefetch_stages may force a
 *   configuration that has grouped kernels (see gemm_mkl_config_name) and its
 *   depth; split_k > 1 or any flag is NOT_AVAILABLE (groups are never split).
 *
 * Rows of K elements that are not a multiple of 16 bytes, or an A or B off a
 * 16-byte boundary, are first copied into zero-padded rows of Kp elements (K
 * rounded up to 16 bytes) in the workspace: opts->workspace, which must then
 * hold the copies (A: total_m * Kp, B: G * N * Kp elements, each rounded up
 * to 256 bytes, A first), or the library's internal one.
 *
 * Returns GEMM_MKL_STATUS_OK (also for G, total_m or N equal to 0: no
 * launch), INVALID_VALUE (negative sizes, G > 65536, total_m >= 2^31, null or
 * element-misaligned pointers, a C or caller workspace sharing bytes with
 * another argument), UNSUPPORTED_DTYPE / _EPILOGUE, WORKSPACE (a
 * caller workspace too small for the repacked operands), NOT_AVAILABLE (no
 * configuration fits) or HIP_ERROR.  Ownership as for gemm_mkl.
 */
int gemm_mkl_grouped(const void *A, const void *B, void *C, const int32_t *offs,
                     int64_t G, int64_t total_m, int64_t N, int64_t K,
                     int dtype, int epilogue, void *stream,
                     const gemm_mkl_opts *opts);

/*
 * RMSNorm over the last axis, the row reduction that "一个可定制的编译器，用于为
 * AI模型生成高效的融合GPU内核" lowers from torch.nn.RMSNorm (its Loop IR and
 * generated kernel): for every row r and column j
 *
 *   y[r][j] = (x[r][j] * rsqrt(sum_j' x[r][j']^2 * (1/hidden) + eps)) * weight[j]
 *
 * x:      device pointer, [rows][hidden], hidden contiguous.
 * weight: device pointer to hidden elements, or NULL for no weight (y = x * rsqrt(...)).
 * y:      device pointer, [rows][hidden]; may equal x (in place); any other
 *         byte shared with x or weight is INVALID_VALUE.
 * x, weight and y share dtype (GEMM_MKL_F32/F16/BF16); the sum, rsqrt and
 * products run in fp32 and the result is rounded once (round to nearest even)
 * to the dtype.  eps must be finite and >= 0.  The squares are summed in an
 * order fixed by hidden and the kernel variant: results are bitwise
 * reproducible.
 *
 * Returns GEMM_MKL_STATUS_OK (also for rows or hidden equal to 0: no launch),
 * INVALID_VALUE (negative sizes, hidden >= 2^31, size overflow, eps negative,
 * NaN or infinite, null x or y for a non-empty problem, element-misaligned
 * pointers, y partly over x or over the weight), UNSUPPORTED_DTYPE or HIP_ERROR.  Enqueued on `stream` (a
 * hipStream_t, NULL = default stream); nothing is allocated and the call does
 * not synchronise.
 */
int gemm_mkl_rms_norm(const void *x, const void *weight, void *y,
                      int64_t rows, int64_t hidden, float eps,
                      int dtype, void *stream);

/* gemm_mkl_rms_norm with a forced kernel variant (-1 = automatic; see
 * gemm_mkl_rms_norm_variant_name).  Variant 0 is the general kernel (any
 * hidden, element-aligned pointers); the others are vector kernels that need
 * 16-byte aligned x, weight and y, hidden * element size a multiple of 16 and
 * a row no longer than the variant covers: otherwise NOT_AVAILABLE.  A
 * variant outside [-1, gemm_mkl_rms_norm_num_variants()) is INVALID_VALUE. */
int gemm_mkl_rms_norm_ex(const void *x, const void *weight, void *y,
                         int64_t rows, int64_t hidden, float eps,
                         int dtype, void *stream, int variant);

/* The variant gemm_mkl_rms_norm would use for these sizes, given whether x,
 * weight and y are all 16-byte aligned (aligned != 0).  Launches nothing;
 * returns a variant id >= 0 or a negative status. */
int gemm_mkl_rms_norm_variant(int64_t rows, int64_t hidden, int dtype, int aligned);

/* Number of RMSNorm kernel variants, and the name of one (NULL when out of range). */
int gemm_mkl_rms_norm_num_variants(void);
const char *gemm_mkl_rms_norm_variant_name(int variant);

/* The configuration id gemm_mkl_grouped would use for these sizes and options
 * (>= 0, see gemm_mkl_config_name), or a negative status: the checks of
 * gemm_mkl_grouped that need no pointers.  Launches nothing. */
int gemm_mkl_grouped_config(int64_t G, int64_t total_m, int64_t N, int64_t K,
                            int dtype, int epilogue, const gemm_mkl_opts *opts);

/*
 * The plan gemm_mkl_ex would execute for these arguments, without launching
 * anything: chosen configuration id, prefetch depth, split factor, grid size
 * and workspace bytes.  Returns a status like gemm_mkl_ex (argument checks
 * are the same; pointers are not needed).
 */
typedef struct gemm_mkl_plan {
    int32_t config_id;
    int32_t prefetch_stages;
    int32_t split_k;
    int32_t general;          /* 1 if the general kernel is used */
    int64_t grid;             /* workgroups of the main kernel */
    int32_t block_m, block_n, block_k, threads;
    size_t workspace_bytes;   /* 0 when split_k == 1 and not stream-K */
    int32_t streamk;          /* 1 if the stream-K kernel is used (grid = workgroups) */
    int32_t counter_bytes;    /* stream-K: leading workspace bytes holding counters */
    int32_t persistent;       /* 1 if the persistent grid is used (grid = workgroups) */
    int32_t packed;           /* 1 if A and B are first copied into zero-padded,
                                 16-byte aligned rows in the workspace (K * elem
                                 not a multiple of 16 bytes) */
    int32_t fixup;            /* 1 if the split_k pieces of each tile are summed inside
                                 the GEMM kernel (no reduction launch); counter_bytes
                                 then gives its per-tile counter words */
} gemm_mkl_plan;

int gemm_mkl_get_plan(int64_t M, int64_t N, int64_t K, int64_t L,
                      int dtype, int epilogue, const gemm_mkl_opts *opts,
                      gemm_mkl_plan *plan);

/*
 * The tile each workgroup of the plan's data-parallel (or split-K) grid
 * computes, as the kernel derives it from its workgroup id: for workgroup b
 * of the plan's grid, out[4b .. 4b+3] = (batch, K split, tile row, tile
 * column).  The order shows the XCD-aware raster (workgroup b runs on XCD
 * b % 8).  `out` is host memory of `capacity` int32 entries, owned by the
 * caller; it must hold 4 * grid entries (gemm_mkl_get_plan gives the grid).
 * Argument checks as in gemm_mkl_get_plan; NOT_AVAILABLE when the plan uses
 * the general, stream-K or persistent kernel (no such per-workgroup tile),
 * INVALID_VALUE when out is NULL or too small.  For a fix-up plan the entries
 * are (batch, piece, tile row, tile column), all -1 for a workgroup that
 * holds no tile (past the last tile of its XCD's run).  Empty problems write
 * nothing.  Launches nothing.
 */
int gemm_mkl_tile_order(int64_t M, int64_t N, int64_t K, int64_t L,
                        int dtype, int epilogue, const gemm_mkl_opts *opts,
                        int32_t *out, int64_t capacity);

/* Bytes of split-K workspace for the plan of these arguments (0 if none). */
size_t gemm_mkl_workspace_size(int64_t M, int64_t N, int64_t K, int64_t L,
                               int dtype, int split_k);

/* Frees the internal split-K workspaces of every device (call with no GEMM in
 * flight).  Returns GEMM_MKL_STATUS_OK or GEMM_MKL_STATUS_HIP_ERROR. */
int gemm_mkl_release_workspace(void);

/* A static, human-readable description of a status code (never NULL).  For
 * GEMM_MKL_STATUS_HIP_ERROR it names the last HIP error seen by this thread. */
const char *gemm_mkl_status_string(int status);

/* Number of entries in the kernel configuration table, and a static
 * description of entry `id` (NULL if out of range). */
int gemm_mkl_num_configs(void);
const char *gemm_mkl_config_name(int id);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int gemm_mkl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_MKL_H_ */
