/*
 * tg_gemm.h -- C interface of the MI355X (gfx950) tiled half-precision GEMM.
 *
 * The operation is the dense matrix product of the TileLang pages' central
 * example ("TileLang: writing LLM GPU kernels by thinking in tiles", section
 * 2 "The basic idea: a GPU should reuse data", and section 3's listing
 * signature: A is MxK, B is KxN, C is MxN, 16-bit inputs and output with a
 * 32-bit float accumulator), optionally followed by the fused epilogue of
 * "Designing high-performance GPU kernels with TileLang", part 3 "Epilogue
 * fusion": C = GELU(A*B + bias), computed while the product is still in
 * registers.
 *
 *   C[i,j] = epi( sum_k A[i,k] * B[k,j] )          (sum accumulated in fp32)
 *   epi(y) = y                                      TG_EPI_NONE
 *          = y + bias[j]                            TG_EPI_BIAS
 *          = gelu_tanh(y + bias[j])                 TG_EPI_BIAS_GELU_TANH
 *   gelu_tanh(x) = 0.5*x*(1 + tanh(sqrt(2/pi)*(x + 0.044715*x^3)))
 *
 * followed by one round-to-nearest-even conversion to the output format.
 * The order of the fp32 additions is the kernel's; with a bias epilogue the
 * bias may enter the fp32 sum as its first term (y + bias[j] up to that
 * rounding order; exact whenever every partial sum is).
 *
 * Layout and ownership
 *   All matrices are dense, row-major and packed: A has row stride K, B has
 *   row stride N, C has row stride N (no leading-dimension arguments).  A, B,
 *   bias and C are all of `dtype`; bias has N entries and is indexed by the
 *   column j.  All pointers are DEVICE pointers owned by the caller; the
 *   library allocates nothing, keeps no per-call state and never frees.
 *   No alignment is required: aligned pointers and K, N multiples of 8 only
 *   select a faster kernel.
 *
 * Execution
 *   tg_gemm enqueues its kernel on `stream` (a hipStream_t; NULL means the
 *   default stream) and returns without synchronising: TG_OK means
 *   "enqueued".  The call is thread-safe.  Validation happens on the host
 *   before any HIP call, so argument errors never touch the device.
 *
 * Errors (returned, never thrown or aborted)
 *   TG_ERR_INVALID_ARG  a negative M, N or K; an unknown dtype, epilogue or
 *                       path; A or B NULL while M*K or K*N is non-zero; C NULL
 *                       while M*N is non-zero; bias NULL with a bias epilogue
 *                       or non-NULL with TG_EPI_NONE; C overlapping A, B or
 *                       bias.
 *   TG_ERR_UNSUPPORTED  an operand of more than 2^31 - 64 elements (just
 *                       under 4 GiB), a dimension above 2^30, or an explicit path
 *                       (tg_gemm_path) whose shape/alignment requirements the
 *                       arguments do not meet.
 *   TG_ERR_LAUNCH       the HIP runtime reported an error for the launch.
 *
 * Degenerate shapes
 *   M == 0 or N == 0: nothing to compute, TG_OK, no launch.
 *   K == 0: the sum is empty, so C = epi(0), i.e. bias / GELU(bias) / 0.
 */
#ifndef TG_GEMM_H
#define TG_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Every enum below has a last enumerator of INT_MIN (-0x7fffffff - 1): the
 * type is then an int whose every value is a value of the type, so a caller
 * may pass any int and the library's checks (not undefined behaviour)
 * decide what it means.
 */
typedef enum { TG_F16 = 0, TG_BF16 = 1, TG_DTYPE_FORCE_INT = -0x7fffffff - 1 } tg_dtype;

typedef enum {
    TG_EPI_NONE = 0,
    TG_EPI_BIAS = 1,
    TG_EPI_BIAS_GELU_TANH = 2,
    TG_EPILOGUE_FORCE_INT = -0x7fffffff - 1
} tg_epilogue;

typedef enum {
    TG_OK = 0,
    TG_ERR_INVALID_ARG = 1,
    TG_ERR_UNSUPPORTED = 2,
    TG_ERR_LAUNCH = 3,
    TG_STATUS_FORCE_INT = -0x7fffffff - 1
} tg_status;

/*
 * Kernel families.  TG_PATH_AUTO lets the library choose:
 *   TG_PATH_SKINNY         M <= 64 (the decode-shaped product): streams B from
 *                          HBM once; needs K % 8 == 0, N % 4 == 0, A 16-byte
 *                          aligned, B, C and bias 8-byte aligned.  Chosen
 *                          automatically for M <= 16, and for 17 <= M <= 64
 *                          while N <= 16384 (wider B runs faster tiled).
 *   TG_PATH_TILED          MFMA tiles (256x256 by default; see tg_tiles for
 *                          the other sizes and how one is chosen) staged
 *                          through LDS by 16-byte direct loads; any shape
 *                          and alignment as long as A
 *                          and B, each padded to whole tiles, stay below 2 GiB
 *                          less 64 KiB: 2 (M + 256) K and 2 (K + 64) (N + 256)
 *                          both below 2^31 - 65536.  Fastest with K % 8 == 0,
 *                          N % 8 == 0, A, B, C 16-byte and bias 8-byte
 *                          aligned.
 *   TG_PATH_TILED_GENERIC  the same tiling with loads gathered through
 *                          registers and element-granular stores: any shape
 *                          and alignment up to the per-operand limit; chosen
 *                          automatically only for operands too large for
 *                          TG_PATH_TILED.
 *   TG_PATH_NONE           (reported by tg_gemm_plan only) nothing to launch.
 */
typedef enum {
    TG_PATH_AUTO = 0,
    TG_PATH_TILED = 1,
    TG_PATH_TILED_GENERIC = 2,
    TG_PATH_SKINNY = 3,
    TG_PATH_NONE = 4,
    TG_PATH_FORCE_INT = -0x7fffffff - 1
} tg_path;

/*
 * C = epi(A*B [+ bias]) as described above, enqueued on `stream`.
 *   M, N, K   matrix sizes (>= 0)
 *   dtype     format of A, B, bias and C
 *   A         device pointer, M x K, row-major
 *   B         device pointer, K x N, row-major
 *   bias      device pointer, N entries; NULL iff epilogue == TG_EPI_NONE
 *   C         device pointer, M x N, row-major; written, never read
 *   stream    hipStream_t or NULL
 */
tg_status tg_gemm(int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                  const void *A, const void *B, const void *bias, tg_epilogue epilogue,
                  void *C, void *stream);

/*
 * As tg_gemm, but runs the kernel family `path` (TG_PATH_AUTO behaves as
 * tg_gemm).  Returns TG_ERR_UNSUPPORTED when the arguments do not meet the
 * family's requirements listed above.  Meant for tests and benchmarks that
 * compare kernel families on the same inputs.
 */
tg_status tg_gemm_path(tg_path path, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                       const void *A, const void *B, const void *bias, tg_epilogue epilogue,
                       void *C, void *stream);

/*
 * Validates the arguments exactly as tg_gemm does and reports in *path_out
 * the kernel family tg_gemm would launch (TG_PATH_NONE when there is nothing
 * to do).  Pure host code: makes no HIP call, reads no device memory.
 */
tg_status tg_gemm_plan(int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                       const void *A, const void *B, const void *bias, tg_epilogue epilogue,
                       const void *C, tg_path *path_out);

/*
 * Tile configurations of the TG_PATH_TILED family: BM x BN (rows by columns
 * of C per workgroup), the k-extent BK of each pipeline stage, the number of
 * LDS stages and the number of waves per workgroup.  The TileLang pages
 * leave these to the user and tune them per shape ("Designing
 * high-performance GPU kernels with TileLang", "Performance Analysis and
 * Autotuning": a benchmark sweep over block sizes, pipeline stages and
 * thread counts picks the winner, most of all for non-standard dimensions;
 * "TileLang: you write the dataflow, the compiler owns the schedule", "What
 * a tile costs, exactly": the stage count sets the shared-memory footprint;
 * "TileLang: writing LLM GPU kernels by thinking in tiles", section 6: tile
 * recommendation from hardware information and heuristics).  Here every
 * configuration is one instance of the same kernel; TG_TILES_AUTO (what
 * tg_gemm uses) takes the one a cost model built from a measured sweep
 * predicts fastest: the number of rounds of tiles the persistent grid needs
 * on the device's compute units, times the time of one round, a fixed
 * per-tile cost plus K over the configuration's measured per-CU throughput.
 * The 256x256 tile is the most efficient per CU; the smaller ones keep more
 * CUs busy when the output has few 256x256 tiles (the 128x128 tiles run two
 * workgroups per CU).
 *                          BM x BN    BK  stages  waves
 *   TG_TILES_256x256       256x256    32    4       4
 *   TG_TILES_256x128       256x128    32    4       4
 *   TG_TILES_128x256       128x256    32    4       4
 *   TG_TILES_128x128       128x128    32    4       4   (2 per CU)
 *   TG_TILES_256x256_K64   256x256    64    2       4
 *   TG_TILES_256x128_K64   256x128    64    3       4
 *   TG_TILES_128x256_K64   128x256    64    3       4
 *   TG_TILES_128x128_K64   128x128    64    2       4   (2 per CU)
 *   TG_TILES_256x256_W8    256x256    32    4       8   (2 per SIMD, 128x64 each)
 */
typedef enum {
    TG_TILES_AUTO = 0,
    TG_TILES_256x256 = 1,
    TG_TILES_256x128 = 2,
    TG_TILES_128x256 = 3,
    TG_TILES_128x128 = 4,
    TG_TILES_256x256_K64 = 5,
    TG_TILES_256x128_K64 = 6,
    TG_TILES_128x256_K64 = 7,
    TG_TILES_128x128_K64 = 8,
    TG_TILES_256x256_W8 = 9,
    TG_TILES_FORCE_INT = -0x7fffffff - 1
} tg_tiles;

/*
 * As tg_gemm_path(TG_PATH_TILED, ...) with tile configuration `tiles`
 * (TG_TILES_AUTO: the library's choice).  TG_ERR_INVALID_ARG for an unknown
 * configuration, TG_ERR_UNSUPPORTED when the shape is outside the
 * TG_PATH_TILED limit; otherwise the same argument rules, degenerate shapes
 * and results (to the tolerance of fp32 accumulation in a different order;
 * bit-identical on integer-valued inputs) as tg_gemm.  Meant for tests and
 * for tuning sweeps.
 */
tg_status tg_gemm_tiled(tg_tiles tiles, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                        const void *A, const void *B, const void *bias, tg_epilogue epilogue,
                        void *C, void *stream);

/*
 * As tg_gemm_tiled, with the raster of the tiles chosen too: each XCD walks
 * its share of the output tiles group_m tile-rows at a time, column by
 * column, so that the tiles running together share A and B panels in that
 * XCD's L2 (0: the library's choice, 4).  group_m 1..64; other values are
 * TG_ERR_INVALID_ARG.  Results do not depend on group_m.  Meant for tuning
 * sweeps.
 */
tg_status tg_gemm_tiled_grouped(tg_tiles tiles, int group_m, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                                const void *A, const void *B, const void *bias, tg_epilogue epilogue,
                                void *C, void *stream);

/*
 * The configuration TG_TILES_AUTO picks for an M x N x K product on a device
 * with num_cu compute units (num_cu <= 0: 256, an MI355X), in *tiles_out.
 * TG_ERR_INVALID_ARG for negative sizes or a NULL tiles_out.  Pure host code.
 */
tg_status tg_gemm_tiles_plan(int64_t M, int64_t N, int64_t K, int num_cu, tg_tiles *tiles_out);

/*
 * Split-K for the TG_PATH_SKINNY family.  A decode-shaped product (M <= 16)
 * costs what it takes to stream B from HBM once ("TileLang: writing LLM GPU
 * kernels by thinking in tiles", section 2, "A back-of-the-envelope
 * calculation"), and the skinny kernel gives each 64-column slab of B to one
 * workgroup, so a narrow B (N = 4096: 64 slabs) leaves most of a 256-CU
 * device idle, and a slab count that does not divide the CU count (N =
 * 11008: 172 slabs) leaves the rest idle.  Each CU streams at a limited
 * rate of its own, so the time is that of the busiest CU.  The pages have
 * no split-K; this library adds two forms:
 *   even split (splits >= 2): the K range of each slab is divided over
 *     `splits` workgroups;
 *   stream-K (splits = TG_SPLIT_STREAM_K): the 32-k steps of all slabs, slab
 *     after slab, are cut into one equal contiguous range per CU (at most
 *     1024 workgroups, at least 16 steps each), so a workgroup finishes some
 *     slabs and shares the slabs at its range's ends with its neighbours.
 * In both, each workgroup with part of a slab writes its fp32 partial
 * 16 x 64 block to a workspace and counts itself in that slab's counter,
 * and the last to arrive adds the partials in K order, applies the epilogue
 * and stores C.  No workgroup waits for another.
 *
 * tg_gemm_split: as tg_gemm, with the skinny family's K range divided as
 * `splits` says (0: the library's choice, reported by tg_gemm_split_plan for
 * the device of `stream`; 1: no split, no workspace; 2..64 even splits;
 * TG_SPLIT_STREAM_K).  Shapes that do not take the skinny path, those with
 * M > 16 (several row blocks per workgroup, never split) and K = 0 run as in
 * tg_gemm and leave the workspace alone.
 *   workspace        device memory, 16-byte aligned, at least
 *                    tg_gemm_split_workspace_bytes(N, splits) bytes (for
 *                    splits 0, the bytes tg_gemm_split_plan reports; NULL
 *                    allowed when that is 0), not overlapping A, B, bias or
 *                    C.  Its first max(64 KiB, 4 ceil(N / 64) bytes) are
 *                    counters that must be zero before the first call
 *                    (zero-fill the workspace once); every call that
 *                    completes leaves them zero, and partial blocks go
 *                    only after them, so one workspace serves calls of
 *                    every shape with N up to 2^20 (larger N move the
 *                    partials: zero the counters again when N changes).
 *                    Calls that may run at the same time (other streams)
 *                    need workspaces of their own.
 *   workspace_bytes  its size in bytes.
 * TG_ERR_INVALID_ARG for splits outside TG_SPLIT_STREAM_K..64 or a workspace
 * that is missing, too small, misaligned or overlapping; otherwise the
 * argument rules and results of tg_gemm (to the tolerance of fp32
 * accumulation in another order; bit-identical on integer-valued inputs,
 * and the same for every call with the same splits on the same device).
 */
#define TG_SPLIT_STREAM_K (-1)

tg_status tg_gemm_split(int splits, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                        const void *A, const void *B, const void *bias, tg_epilogue epilogue,
                        void *C, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Workspace bytes tg_gemm_split needs for N columns and `splits` splits:
 * 0 for splits 0 and 1 (for 0, ask tg_gemm_split_plan); for
 * TG_SPLIT_STREAM_K, enough for any device (up to 1024 workgroups); -1 for
 * N outside 0..2^30 or splits outside TG_SPLIT_STREAM_K..64.  Pure host code.
 */
int64_t tg_gemm_split_workspace_bytes(int64_t N, int splits);

/*
 * The split mode tg_gemm_split(0, ...) uses for an M x N x K product on a
 * device with num_cu compute units (num_cu <= 0: 256), in *splits_out (1 for
 * M > 16 or an empty product; 2..64; or TG_SPLIT_STREAM_K), and the
 * workspace bytes it needs there, in *workspace_bytes_out.  The even count
 * is the largest with slabs x splits at most num_cu (one round of
 * workgroups; a second costs more than splitting gains) and at least 16
 * 32-k steps per workgroup; stream-K replaces it where a cost model fitted
 * to MI355X times predicts it faster: long K with slabs that leave CUs idle
 * (16 x 11008 x 11008), not the decode shape 16 x 11008 x 4096, where the
 * exchange of partial sums costs more than the idle CUs would gain.
 * TG_ERR_INVALID_ARG for negative or too large sizes or NULL outputs.  Pure
 * host code.
 */
tg_status tg_gemm_split_plan(int64_t M, int64_t N, int64_t K, int num_cu, int *splits_out,
                             int64_t *workspace_bytes_out);

/*
 * Split-K of the skinny family without any workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): tg_gemm_split with the
 * workspace taken from a static device array inside the library,
 * TG_SCRATCH_BYTES bytes per GPU, held until the process ends.  The library
 * allocates and frees nothing in this call.
 *   splits   as for tg_gemm_split (0: tg_gemm_split_plan's choice; 1: no
 *            split; 2..64; TG_SPLIT_STREAM_K).  Shapes that do not take the
 *            skinny path, M > 16, K = 0 and a resolved count of 1 run
 *            exactly as tg_gemm.
 * Limits: ceil(N / 64) x splits (stream-K: workgroups + ceil(N / 64) - 1)
 * at most 1024 (the partial blocks, 4 KiB each) and ceil(N / 64) at most
 * 16384 (the counters), else
 * TG_ERR_UNSUPPORTED; splits outside 0..64 is TG_ERR_INVALID_ARG; the other
 * rules and results are those of tg_gemm_split with the same splits
 * (bit-identical to it).
 * The array is shared by every call on one GPU: calls that may overlap on
 * one GPU (other streams, other threads) race and must not be made; calls
 * on one stream are ordered and safe.  The first call on a device looks the
 * array up (switching the current device for that moment) and enqueues a
 * kernel that zeroes its counters; make it outside graph capture.  Every
 * completed call leaves the counters zero again.
 */
#define TG_SCRATCH_BYTES (4259840)   /* 64 KiB of counters + 4 MiB of partial blocks */

tg_status tg_gemm_split_static(int splits, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                               const void *A, const void *B, const void *bias, tg_epilogue epilogue,
                               void *C, void *stream);

/*
 * Elementwise epilogue steps as passes of their own over a matrix in device
 * memory -- the unfused form of the epilogue that the fourth TileLang page
 * ("Designing high-performance GPU kernels with TileLang", part 3 "Epilogue
 * fusion") measures the fused one against:
 *   TG_EW_BIAS_ADD   Y[m][n] = X[m][n] + bias[n]
 *   TG_EW_GELU_TANH  Y[m][n] = GELU_tanh(X[m][n])    (bias must be NULL)
 * computed in fp32 from the 16-bit inputs and rounded to nearest even once.
 *   M, N    matrix sizes (>= 0); M == 0 or N == 0 is a no-op
 *   dtype   format of X, Y and bias
 *   bias    device pointer, N entries (TG_EW_BIAS_ADD only)
 *   X, Y    device pointers, M x N row-major; Y == X (in place) is allowed,
 *           any other overlap of Y with X or bias is TG_ERR_INVALID_ARG
 *   stream  hipStream_t or NULL
 * Any alignment works; N % 8 == 0 with 16-byte aligned X, Y and bias takes
 * the 16-byte path.  TG_ERR_UNSUPPORTED: M x N above 2^31 - 64 elements.
 */
typedef enum {
    TG_EW_BIAS_ADD = 0,
    TG_EW_GELU_TANH = 1,
    TG_EW_FORCE_INT = -0x7fffffff - 1
} tg_elementwise_op;

tg_status tg_elementwise(tg_elementwise_op op, int64_t M, int64_t N, tg_dtype dtype,
                         const void *bias, const void *X, void *Y, void *stream);

/*
 * The same result as tg_gemm up to rounding, computed unfused: the product
 * without epilogue is written to C, then TG_EW_BIAS_ADD and (for
 * TG_EPI_BIAS_GELU_TANH) TG_EW_GELU_TANH run in place on C -- one, two or
 * three launches, each intermediate rounded to `dtype` in C.  Same arguments
 * and errors as tg_gemm.  A baseline for measuring what fusion saves, not a
 * faster path.
 */
tg_status tg_gemm_unfused(int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                          const void *A, const void *B, const void *bias, tg_epilogue epilogue,
                          void *C, void *stream);

/*
 * Weight-only 4-bit GEMM, the quantized-inference product that the first
 * TileLang page ("TileLang: writing LLM GPU kernels by thinking in tiles",
 * section 5, "Quantized LLM inference") describes: weights stay packed in
 * memory and are dequantized in registers on their way into the product.
 *
 *   C = epi(A * W [+ bias]),   W[k][n] = (q[k][n] - 8) * scales[k / group][n]
 *
 * with q[k][n] in 0..15.  The weights are first packed once into the layout
 * the kernel streams (tg_w4_pack); the product then reads K*N/2 bytes of
 * weights instead of 2*K*N.  fp32 accumulation; each group's scale multiplies
 * the fp32 partial product of that group, and the integers q - 8 enter the
 * matrix instruction exactly.
 */

/* Bytes of the packed weights of a K x N matrix: 32 * K * ceil(N / 64)
 * (N padded to 64 columns); -1 unless K >= 0, N >= 0 and K % 32 == 0. */
int64_t tg_w4_packed_bytes(int64_t K, int64_t N);

/*
 * Packs q (device, K x N bytes row-major, one value 0..15 per byte; higher
 * bits are ignored) into `packed` (device, tg_w4_packed_bytes(K, N) bytes,
 * 16-byte aligned), enqueued on `stream`.  Errors: INVALID_ARG for K % 32 != 0,
 * negative sizes, null pointers with K*N > 0, packed misaligned or
 * overlapping q; UNSUPPORTED above 2^31 - 64 packed or unpacked bytes.
 */
tg_status tg_w4_pack(int64_t K, int64_t N, const void *q, void *packed, void *stream);

/*
 * The product itself.  A (M x K), scales (K/group x N), bias (N), C (M x N)
 * are 16-bit values of `dtype`, row-major, device pointers, any 2-byte
 * alignment; packed as written by tg_w4_pack for the same K and N.
 * group is 32, 64, 128 or 256 and divides K.  Any M (the kernel handles 16
 * rows per workgroup; best for M <= 16).  Same epilogue, bias and degenerate
 * shape rules as tg_gemm (K == 0 gives epi(0 + bias)); C must not overlap
 * any input.  UNSUPPORTED when an operand exceeds 2^31 - 64 elements or
 * bytes, or M exceeds 16 * 65535.
 */
tg_status tg_gemm_w4(int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void *A, const void *packed,
                     const void *scales, int64_t group, const void *bias, tg_epilogue epilogue, void *C,
                     void *stream);

/*
 * Split-K of the 4-bit product, as tg_gemm_split is for the skinny kernel
 * (same workspace protocol, not on the pages): the scale groups of each
 * output block (16 rows x 64 columns) are divided over `splits` workgroups
 * (0: the library's choice, tg_gemm_w4_split_plan for the device of
 * `stream`; 1: no split; at most 64).  workspace: device memory, 16-byte
 * aligned, at least tg_gemm_w4_split_workspace_bytes(M, N, splits) bytes,
 * overlapping no operand, its first max(64 KiB, 4 ceil(M / 16) ceil(N / 64)
 * bytes) zero before the first call and left zero by every completed call
 * (the counters, as for tg_gemm_split); one per stream.  TG_ERR_INVALID_ARG for splits outside 0..64 or a missing, small,
 * misaligned or overlapping workspace; otherwise the rules and results of
 * tg_gemm_w4 (to the tolerance of fp32 accumulation in another order;
 * bit-identical on integer-valued inputs and from call to call).
 */
tg_status tg_gemm_w4_split(int splits, int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void *A,
                           const void *packed, const void *scales, int64_t group, const void *bias,
                           tg_epilogue epilogue, void *C, void *workspace, int64_t workspace_bytes,
                           void *stream);

/* Workspace bytes of tg_gemm_w4_split for an M x N output and `splits`
 * splits (0 for splits <= 1; -1 for sizes outside the limits of tg_gemm_w4
 * or splits outside 0..64).  Pure host code. */
int64_t tg_gemm_w4_split_workspace_bytes(int64_t M, int64_t N, int splits);

/*
 * The split count tg_gemm_w4_split(0, ...) uses on a device with num_cu
 * compute units (num_cu <= 0: 256) and its workspace bytes: the largest
 * count with ceil(M / 16) ceil(N / 64) splits at most num_cu and at least 8
 * scale groups (one per wave) per workgroup; 1 for an empty product.
 * TG_ERR_INVALID_ARG for invalid sizes or group, or NULL outputs.  Pure
 * host code.
 */
tg_status tg_gemm_w4_split_plan(int64_t M, int64_t N, int64_t K, int64_t group, int num_cu, int *splits_out,
                                int64_t *workspace_bytes_out);

/*
 * Attention forward, the fused kernel the TileLang pages build around the same
 * tiles ("TileLang: writing LLM GPU kernels by thinking in tiles", section 5,
 * "FlashAttention"; "TileLang: you write the dataflow, the compiler owns the
 * schedule", "FlashAttention, in tiles"):
 *
 *   O[b][i][h][:] = sum_j softmax_j(scale * Q[b][i][h][:] . K[b][j][h][:]) V[b][j][h][:]
 *
 * over the visible keys j: all j < Sk, or with causal != 0 (which needs
 * Sq == Sk) the keys j <= i.  The score matrix is never stored: key/value
 * blocks stream through on-chip memory with an online softmax, fp32 scores
 * and accumulation, and the probabilities rounded to `dtype` on their way
 * into the second product.
 *   batch, Sq, Sk, heads  sizes (>= 0); head_dim must be 128
 *   Q, O      device pointers, [batch][Sq][heads][head_dim] row-major (BSHD)
 *   K, V      device pointers, [batch][Sk][heads][head_dim]
 *   scale     softmax scale > 0, or 0 for 1/sqrt(head_dim)
 *   stream    hipStream_t or NULL
 * Any 2-byte alignment.  A query with no visible key (Sk == 0) gets O = 0.
 * Errors: INVALID_ARG for negative sizes, a bad dtype, causal with Sq != Sk,
 * a negative or non-finite scale, null pointers where data is read or
 * written; UNSUPPORTED for head_dim != 128, more than 65535 heads or
 * batches, or Q/O or K/V (padded by a block of queries or keys) beyond 2 GiB
 * less 64 KiB; then INVALID_ARG for O overlapping Q, K or V.
 */
tg_status tg_attention_fwd(int64_t batch, int64_t Sq, int64_t Sk, int64_t heads, int64_t head_dim, tg_dtype dtype,
                           const void *Q, const void *K, const void *V, int causal, float scale, void *O,
                           void *stream);

/* Static, human-readable name of a status code ("TG_OK", ...). */
const char *tg_status_string(tg_status status);

/* Static version string of the library. */
const char *tg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TG_GEMM_H */
