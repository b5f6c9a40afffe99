/*
 * tdi8.h -- C ABI of the MI355X (gfx950) tiled int8 matrix-multiply library.
 *
 * Operation.  C = A x B with signed int8 A (M x K) and B (K x N) and int32 C
 * (M x N): C[i][j] = sum_k A[i][k] * B[k][j], accumulated in int32.  This is
 * the product the TPU notes describe being fed, in passes, through a 256 x 256
 * INT8 multiply-accumulate array ("Motivation for and Evaluation of the First
 * Tensor Processing Unit" notes, sections "TPU介绍" and "TPU使用的技术"), and
 * the matrix multiply whose tiling the CUDA tutorial analyses ("CUDA编程实践",
 * section 3).  The kernel that runs is chosen per problem size from a table
 * of compiled tile configurations, as the system of patent application
 * CN114238853A does (claim 7: one kernel compiled per configuration, the
 * configuration parameters being the kernel's template parameters, the best
 * one selected at run time from the input size).
 *
 * Results are exact: every partial sum is an int32 and integer addition is
 * associative, so the bytes of C do not depend on the tiling, the K split or
 * the order of accumulation.  C is defined modulo 2^32 (two's-complement
 * wrap); no wrap occurs while K <= 131071.
 *
 * Memory.  A, B and C are device pointers (hipMalloc'd, or a torch tensor's
 * data_ptr()) owned by the caller.  The library allocates nothing and keeps no
 * pointer after a call returns.  A and B are read only.  Only the window
 * C[0:M, 0:N] is written; bytes of C's rows beyond column N (row padding up to
 * ldc) are never touched.
 *
 * Layouts (all leading dimensions in elements):
 *   A  row-major:        A(i,k) at A[i*lda + k],  lda >= K
 *   B  row-major:        B(k,j) at B[k*ldb + j],  ldb >= N   (gemm_s8s8s32)
 *   B  column-major:     B(k,j) at B[j*ldb + k],  ldb >= K   (gemm_s8s8s32_bt)
 *   C  row-major:        C(i,j) at C[i*ldc + j],  ldc >= N
 * Any pointer alignment and any leading dimension are accepted; 16-byte
 * aligned operands (lda, ldb multiples of 16, ldc of 4) with K a multiple of
 * 16 (and, for row-major B, N a multiple of 16) take the unpredicated fast
 * kernels, whatever the other sizes: rows, columns and K positions past the
 * operands read a 16-byte zero block and stores past M or N are masked.  The
 * rest take the predicated tail kernels.
 *
 * Streams and errors.  Calls are asynchronous: work is enqueued on `stream`
 * (0 = the null stream) and the call returns without waiting.  All argument
 * checks run on the host before anything is enqueued; a call that returns an
 * error has enqueued nothing.  A failed kernel launch returns TDI8_ERR_HIP
 * and tdi8_last_hip_error() gives the hipError_t.  Faults inside a kernel
 * surface at the caller's next synchronisation.  Nothing is printed.
 *
 * Threads.  Initialisation (device query, per-kernel occupancy) happens once
 * per device on first use and is thread safe; afterwards every entry point is
 * re-entrant.  Calls on one stream execute in order.
 */
#ifndef TDI8_H
#define TDI8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same opaque handle type as HIP's own declaration. */
typedef struct ihipStream_t *hipStream_t;

typedef enum {
    TDI8_OK = 0,
    TDI8_ERR_INVALID_VALUE = -1,     /* M, N or K < 0, or a leading dimension too small */
    TDI8_ERR_NULL_POINTER = -2,      /* a pointer the call must dereference is NULL */
    TDI8_ERR_ALIASING = -3,          /* C's window overlaps the bytes of A or B that are read */
    TDI8_ERR_UNSUPPORTED_DEVICE = -4,/* the current device is not gfx950 */
    TDI8_ERR_BAD_CONFIG = -5,        /* unknown configuration id, or it cannot run this shape */
    TDI8_ERR_HIP = -6                /* a HIP runtime call failed; see tdi8_last_hip_error() */
} tdi8_status;

/* Route by which a configuration is reached in the selection. */
typedef enum {
    TDI8_ROUTE_GENERAL = 0,   /* survived the fill-the-compute-units step */
    TDI8_ROUTE_FALLBACK = 1,  /* reuse-1 fallback of the fill step */
    TDI8_ROUTE_SKINNY = 2     /* fallback with M small enough for the skinny family */
} tdi8_route;

/* C = A x B, A row-major M x K, B row-major K x N, C row-major M x N.
 * M == 0 or N == 0: nothing is enqueued.  K == 0: the C window is set to 0.
 * The configuration is select_tile_config's, with one exception: when the
 * operands take the predicated kernels (see above) with column-major B and
 * the selected tiles number fewer than the compute units, the reuse-1
 * configuration with the most tiles, at most one per compute unit, runs
 * instead (the selection relies on the K split to fill the compute units,
 * which the predicated kernels do not have; gemm_plan reports the one that
 * runs).  Returns TDI8_OK or a negative tdi8_status. */
int gemm_s8s8s32(int M, int N, int K, const int8_t *A, int lda, const int8_t *B, int ldb,
                 int32_t *C, int ldc, hipStream_t stream);

/* Same as gemm_s8s8s32 with B column-major: B(k,j) at B[j*ldb + k], ldb >= K
 * (B stored N x K with K contiguous, as inference weights usually are).  This
 * is the operand order of a convolution lowered to a matrix product in the
 * contest write-up ("先导杯比赛回顾", 卷积转化 and 多批次展开的 Im2col 方法):
 * the filter bank, one row of reduction values per output channel, is the
 * right-hand operand with the reduction dimension contiguous, the layout
 * that write-up transposes its NCHW data into (NCHW布局空间连续性不佳,
 * NCHW_2_NHWC) so that the dimension summed over lies contiguously. */
int gemm_s8s8s32_bt(int M, int N, int K, const int8_t *A, int lda, const int8_t *B, int ldb,
                    int32_t *C, int ldc, hipStream_t stream);

/* Same product computed with a given configuration id instead of the
 * selected one (b_col_major selects the B layout).  Patent application
 * CN114238853A, claim 7: the system compiles one kernel per tiling
 * configuration, the configuration's parameters being the kernel's template
 * parameters, and runs the one the selection picks; this entry point runs a
 * compiled configuration by its id, bypassing the selection.  Any general
 * configuration runs any shape; a skinny configuration needs M <= its block
 * height times 65535 (TDI8_ERR_BAD_CONFIG otherwise).  Arguments, layouts,
 * ownership and errors as for gemm_s8s8s32; config_id outside
 * 0 .. tile_config_count()-1 gives TDI8_ERR_BAD_CONFIG.  For tests and the
 * bench, which sweep every compiled configuration. */
int gemm_s8s8s32_with_config(int config_id, int b_col_major, int M, int N, int K,
                             const int8_t *A, int lda, const int8_t *B, int ldb,
                             int32_t *C, int ldc, hipStream_t stream);

/* Configuration id that gemm_s8s8s32 / gemm_s8s8s32_bt use for an M x K by
 * K x N product on the current device (>= 0), or a negative tdi8_status.
 * The five steps of patent application CN114238853A claim 1 (claims 2-6 give
 * the details): enumerate the compiled configurations; keep those whose
 * register-limited active threads per compute unit reach the threshold;
 * keep those launching at least (compute units x resident blocks per compute
 * unit) blocks, or, if none does, every configuration reduced to reuse 1
 * (then, for M <= 32 or else N <= 32, the skinny family: the smallest block
 * height >= M, or width >= N, then the smallest extent along the other side
 * among those launching a block per compute unit); keep the largest compute-to-memory
 * ratio BM*BN/(BM+BN); keep the fewest rounds of resident blocks; first in
 * table order.  Host only; pure after the first call's initialisation. */
int select_tile_config(int M, int N, int K);

/* Description of one compiled configuration: the tiling tuple the claims of
 * patent application CN114238853A select over (claim 2: the thread split
 * block_m_threads = waves_m * mfma_m and block_n_threads = waves_n * mfma_n;
 * claims 4 and 5: the per-wave repeats m_tiles and n_tiles, the block tile
 * block_m x block_n and the K depth block_k; claim 6: the registers each
 * thread uses, the shared memory (LDS) each block uses and the resulting
 * resident blocks per compute unit, block_per_cu).  Register and LDS figures
 * are those of the configuration's column-major-B unpredicated kernel, read
 * by the build from the compiled code object's metadata. */
typedef struct {
    int id;
    int family;          /* 0 general tiled kernel, 1 skinny (split-K across waves) kernel */
    int mfma_m, mfma_n, mfma_k;  /* matrix-core instruction shape */
    int waves_m, waves_n, waves_k;
    int m_tiles, n_tiles;        /* per-wave instruction repeats (the claims' data reuse) */
    int block_m, block_n, block_k;
    int stages;          /* LDS stages of the unpredicated column-major-B kernel */
    int threads;
    int lds_bytes;       /* static LDS per block of that kernel */
    int vgprs;           /* architectural vector registers per lane of that kernel (rounded up
                            to a multiple of 4 when accumulation registers follow them) */
    int agprs;           /* accumulation vector registers per lane of that kernel (the
                            compiler keeps matrix-core accumulators in either file); the
                            lane's allocation spans vgprs + agprs registers */
    int blocks_per_cu;   /* resident blocks per compute unit, from the runtime occupancy query
                            on the current device (0 before a gfx950 device is seen) */
    int reuse1_id;       /* configuration with the same thread split and m_tiles = n_tiles = 1 */
    int excluded;        /* 1: its reuse scheme (family, m_tiles, n_tiles) was excluded by the
                            performance test of claim 3 (second alternative); the selection drops
                            it at step 2, gemm_s8s8s32_with_config still runs it */
    int sgprs;           /* scalar registers per wave of that kernel */
} tdi8_tile_config;

/* Number of compiled configurations; ids are 0 .. count-1. */
int tile_config_count(void);

/* Copies the description of configuration `id` into *out (caller-owned).
 * Everything but blocks_per_cu is static and needs no device; blocks_per_cu
 * is filled once a gfx950 device has been initialised (0 otherwise).
 * Returns TDI8_OK, TDI8_ERR_BAD_CONFIG (unknown id) or TDI8_ERR_NULL_POINTER. */
int tile_config_info(int id, tdi8_tile_config *out);

/* Hardware description used by the selection. */
typedef struct {
    int num_cu;                /* compute units */
    int max_threads_per_block;
    int min_active_threads;    /* claim-3 threshold on register-limited active threads per CU */
    int skinny_max_m;          /* largest M (or, for larger M, N) routed to the skinny family; 0: none */
} tdi8_hw_info;

typedef struct {
    int id;
    int route;                 /* tdi8_route */
    int survivors[5];          /* candidates left after steps 1..5 */
} tdi8_selection;

/* The selection of select_tile_config on explicit hardware: `blocks_per_cu`
 * holds one entry per configuration id (tile_config_count() entries).  Host
 * only, needs no device; used to test the selection on described hardware.
 * Returns the id (>= 0) or a negative tdi8_status; fills *out when non-NULL. */
int select_tile_config_for(int M, int N, int K, const tdi8_hw_info *hw,
                           const int *blocks_per_cu, tdi8_selection *out);

/* K slices the gemm entry points use with configuration `config_id` for an
 * M x K by K x N product on a device of `num_cu` compute units, when the
 * operands take the unpredicated path (16-byte aligned pointers, lda and ldb
 * multiples of 16, ldc of 4, K a multiple of 16, and with row-major B N
 * too); other operands are never split.  Splitting K with integer atomics is
 * the contest write-up's "Split K" paragraph, added after the five steps of
 * the selection: counting the partial tiles at the ends of M and N, while
 * the tiles times twice the slices still fit one block per compute unit, and
 * K over twice the slices is still at least eight K tiles, the slices double.
 * Slices are whole 16-byte chunks of K, differing by at most one; when M, N
 * and every slice are whole tiles the whole-tile form runs, else the edge
 * form.  1 = no split (always for the skinny family).
 * A split call enqueues two kernels on the stream: one zeroes the C window,
 * the other adds every slice's partial sums into it; the result is the same
 * bytes as without the split (integer addition in any order).  Host only,
 * needs no device.  Returns >= 1 or a negative tdi8_status.
 *
 * A skinny configuration with row-major B (gemm_s8s8s32), 16-byte aligned
 * operands, N and K multiples of 16 and N a multiple of 128 or above 256,
 * also enqueues two kernels: each block
 * covers 128 columns (the last ones may end at N) over one of G = 128 /
 * block width slices of K (whole 128-byte lines of every B row it reads),
 * adding into the zeroed C window.  Its K split is
 * a property of the row-major form and is not what this function reports. */
int tile_config_split_k(int config_id, int M, int N, int K, int num_cu);

/* Kernel forms a gemm call can run (gemm_plan). */
typedef enum {
    TDI8_FORM_NONE = 0,             /* M == 0 or N == 0: nothing is enqueued */
    TDI8_FORM_PREDICATED = 1,       /* register-staged tiled kernel: any K, alignment, leading dims */
    TDI8_FORM_PIPELINED = 2,        /* LDS-DMA pipelined kernel, whole tiles */
    TDI8_FORM_PIPELINED_EDGE = 3,   /* the same for sizes that end inside a tile */
    TDI8_FORM_SPLIT = 4,            /* zero fill, then the K split of the pipelined kernel (whole tiles) */
    TDI8_FORM_SPLIT_EDGE = 5,       /* zero fill, then the K split of its edge form */
    TDI8_FORM_SKINNY_DMA = 6,       /* skinny kernel fed by LDS DMA (either B layout) */
    TDI8_FORM_SKINNY_PREDICATED = 7,/* skinny kernel with masked register loads */
    TDI8_FORM_SKINNY_ROW_GROUPS = 8,/* zero fill, then the row-major-B column groups of a skinny tile */
    TDI8_FORM_PREDICATED_PREFETCH = 9, /* the predicated kernel with two K tiles of loads in flight:
                                       * column-major B, at most one block per compute unit */
    TDI8_FORM_PERSISTENT = 10       /* persistent whole-tile kernel: a fixed grid walks the tiles;
                                       run only by gemm_s8s8s32_persistent, so gemm_plan, which
                                       describes the other gemm calls, never reports it */
} tdi8_form;

typedef struct {
    int config_id;   /* configuration that runs (-1 with TDI8_FORM_NONE and no id given) */
    int form;        /* tdi8_form */
    int splits;      /* K slices (column groups for TDI8_FORM_SKINNY_ROW_GROUPS); 1 = none */
    int kernels;     /* kernels enqueued: 2 when a zero fill runs first, else 1 (0 for NONE) */
    int grid_x, grid_y, threads;  /* launch shape of the product kernel */
} tdi8_plan;

/* What a gemm call with these arguments would enqueue on the current device,
 * without enqueueing anything: the configuration (config_id -1: the
 * selection's, as gemm_s8s8s32 / gemm_s8s8s32_bt; else that id, as
 * gemm_s8s8s32_with_config), the kernel form and its launch shape.  Patent
 * application CN114238853A, claim 7: at run time the input size decides the
 * configuration and its compiled kernel; the launch wrappers of the contest
 * write-up ("先导杯比赛回顾", NCHW_2_NHWC and 多批次展开的 Im2col 方法)
 * derive the grid from the sizes before launching.  The form depends on the
 * sizes and on the alignment of the pointers and leading dimensions, so the
 * pointers are the ones the call would pass (they are not dereferenced).
 * Same argument checks and status codes as the gemm call; *out is caller
 * owned and written only on TDI8_OK.  One decision serves the call and this
 * query, so the plan is what runs.  Host only; initialises the device. */
int gemm_plan(int config_id, int b_col_major, int M, int N, int K, const int8_t *A, int lda, const int8_t *B,
              int ldb, const int32_t *C, int ldc, tdi8_plan *out);

/* Same product in the persistent form of a general configuration's
 * whole-tile kernel: `blocks` blocks (0: as many as the device holds at once,
 * the compute units times the persistent kernel's resident blocks per unit,
 * rounded down to a multiple of 8; any value is capped at the tile count)
 * each walk the tiles blocks apart in the block-to-tile order of the other
 * forms, which groups the tiles resident on one XCD into a compact region
 * (the contest write-up "先导杯比赛回顾", Swizzle 线程块映射: block order
 * chosen for cache reuse; 矩阵维度高度不均衡: flat waves of blocks lose it).
 * A block's K tiles form one load stream across its tiles, and each finished
 * tile is stored from the accumulation registers while the next tile's
 * matrix work runs, so the C write of one tile overlaps the next one's
 * product.  config_id -1 takes the selection's configuration.  Needs whole
 * tiles of that configuration (M, N, K multiples of its block_m, block_n,
 * block_k), A, B and C 16-byte aligned, lda and ldb multiples of 16 and ldc
 * a multiple of 4; otherwise, or for a skinny configuration, returns
 * TDI8_ERR_BAD_CONFIG and enqueues nothing.  blocks < 0 gives
 * TDI8_ERR_INVALID_VALUE; M == 0 or N == 0 enqueues nothing and returns
 * TDI8_OK.  Arguments, layouts, ownership and the other errors as for
 * gemm_s8s8s32_with_config.  The result is bit-identical to
 * the other forms' (integer sums). */
int gemm_s8s8s32_persistent(int config_id, int b_col_major, int M, int N, int K, const int8_t *A, int lda,
                            const int8_t *B, int ldb, int32_t *C, int ldc, int blocks, hipStream_t stream);

/* ---- int8 2-D convolution (implicit GEMM on the same kernels) ----------------
 *
 * y = conv2d(x, w) with zero padding, stride and dilation: for every image n,
 * output position (p, q) and filter k,
 *   y[n][p][q][k] = sum over r < R, s < S, c < C of
 *                   x[n][p*stride_h + r*dil_h - pad_h][q*stride_w + s*dil_w - pad_w][c] * w[k][r][s][c],
 * taps outside the image contributing 0, accumulated exactly in int32 (mod
 * 2^32 as for the matrix product).  The input position of a tap is the one
 * the contest write-up's im2col kernel uses ("先导杯比赛回顾", 多批次展开的
 * Im2col 方法), and the convolution is computed as the matrix product it
 * lowers to (卷积转化) without materialising that matrix: M = N*P*Q output
 * pixels, N = K filters, reduction R*S*C, the filters being the column-major
 * B operand.
 *
 * Layouts (dense, no padding between rows): x is N x H x W x C (NHWC), w is
 * K x R x S x C (KRSC), y is N x P x Q x K with P = conv2d_output_extent(H,
 * R, pad_h, stride_h, dil_h) and Q likewise.  The caller owns all three
 * (device memory); the library allocates nothing and keeps no pointer.
 * Requirements: y 4-byte aligned; R, S, stride and dilation >= 1, padding
 * >= 0; any channel count C and any alignment of x and w.  With C a multiple
 * of 16 and x and w 16-byte aligned, every 16-byte chunk of the lowered
 * matrix is 16 channels of one tap and goes to LDS by DMA; otherwise (the
 * first layer of a network, C = 3: reduction 27 for 3 x 3 filters) the rows
 * are gathered into registers, a slower form with the same result: with
 * dil_w = 1 a filter row's S*C bytes lie contiguously in the image and are
 * read in 16-byte pieces, else byte by byte.  Errors, all found on the host before anything is enqueued:
 * TDI8_ERR_INVALID_VALUE (a size, y's alignment, or N*P*Q or R*S*C above
 * INT_MAX),
 * TDI8_ERR_NULL_POINTER, TDI8_ERR_ALIASING (y overlaps x or w),
 * TDI8_ERR_UNSUPPORTED_DEVICE, TDI8_ERR_HIP.  N*P*Q == 0 or K == 0 enqueues
 * nothing; C == 0 writes zeros.  Asynchronous on `stream`.  The tile
 * configuration is the selection's for the (N*P*Q) x (R*S*C) by (R*S*C) x K
 * product, from the general family only. */
int conv2d_s8s8s32_nhwc(int N, int H, int W, int C, int K, int R, int S,
                        int pad_h, int pad_w, int stride_h, int stride_w, int dil_h, int dil_w,
                        const int8_t *x, const int8_t *w, int32_t *y, hipStream_t stream);

/* The same with a given general configuration (TDI8_ERR_BAD_CONFIG for a
 * skinny one); for tests and the bench. */
int conv2d_s8s8s32_nhwc_with_config(int config_id, int N, int H, int W, int C, int K, int R, int S,
                                    int pad_h, int pad_w, int stride_h, int stride_w, int dil_h, int dil_w,
                                    const int8_t *x, const int8_t *w, int32_t *y, hipStream_t stream);

/* Configuration id conv2d_s8s8s32_nhwc uses on the current device, or a
 * negative status.  Host only. */
int conv2d_select_config(int N, int H, int W, int C, int K, int R, int S,
                         int pad_h, int pad_w, int stride_h, int stride_w, int dil_h, int dil_w);

/* Output extent along one axis: (H + 2 pad - dil (R - 1) - 1) / stride + 1,
 * or 0 when the dilated filter does not fit; a negative status for invalid
 * arguments.  Host only, no device needed. */
int conv2d_output_extent(int H, int R, int pad, int stride, int dil);

/* The host-side checks of conv2d_s8s8s32_nhwc (no device needed). */
int conv2d_validate(int N, int H, int W, int C, int K, int R, int S,
                    int pad_h, int pad_w, int stride_h, int stride_w, int dil_h, int dil_w,
                    const int8_t *x, const int8_t *w, const int32_t *y);

/* Host-side argument check shared by every gemm entry point (no device
 * needed): returns TDI8_OK or the status the entry point would return. */
int tdi8_validate(int b_col_major, int M, int N, int K, const int8_t *A, int lda,
                  const int8_t *B, int ldb, const int32_t *C, int ldc);

/* Static string for a status code (never NULL; "unknown status" for a value
 * outside tdi8_status; the caller must not free it).  The contest write-up's
 * launch wrappers ("先导杯比赛回顾", NCHW_2_NHWC and 多批次展开的 Im2col 方法)
 * read hipGetLastError after each launch and print its error string; a
 * library prints nothing, so the status code and this text take its place. */
const char *tdi8_status_string(int status);

/* hipError_t of the last failed HIP call made by this thread (0 if none):
 * the error those launch wrappers obtain from hipGetLastError, kept per
 * thread for the caller after an entry point returned TDI8_ERR_HIP. */
int tdi8_last_hip_error(void);

/* Identity of the GPU code compiled into this library: the first 16 hex
 * digits of the SHA-256 of the gfx950 code objects of every configuration,
 * in configuration order (static string; the caller must not free it).  Two
 * builds report the same value exactly when their kernels are the same
 * machine code, so a measurement taken on one build (a counter pass, a
 * kernel trace) can record it and be matched against the library that runs
 * later.  Not part of the pages' method: a build identity for measurements. */
const char *tdi8_kernel_code_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* TDI8_H */
