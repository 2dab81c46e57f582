// tg_gemm_host.hip -- the C interface (include/tg_gemm.h): argument checks,
// choice of kernel family and the launch on the caller's stream.
//
// Argument checks are plain host arithmetic: no HIP call, no device memory
// access and no allocation, so invalid arguments never reach the device.  The
// only state is a per-device cache of the compute-unit count (one HIP query
// per device, stored atomically), so concurrent calls need no locking.
#include "tg_gemm.h"
#include "tg_launch.h"

#include <atomic>
#include <math.h>
#include <mutex>
#include <stdint.h>

#define TG_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

// Per operand: kernels address operands with 32-bit byte offsets and keep
// offsets of at least 2^32 - 32 for "out of range", so operands stay below that.
constexpr int64_t kMaxElements = (int64_t(1) << 31) - 64;
constexpr int64_t kMaxDim = int64_t(1) << 30;

bool aligned(const void *p, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

// Number of elements of an r x c operand, or -1 if it exceeds kMaxElements.
int64_t elements(int64_t r, int64_t c) {
    if (r == 0 || c == 0)
        return 0;
    if (r > kMaxElements / c)
        return -1;
    return r * c;
}

bool overlaps(const void *p, int64_t pbytes, const void *q, int64_t qbytes) {
    if (!p || !q || pbytes <= 0 || qbytes <= 0)
        return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + static_cast<uintptr_t>(qbytes) && b < a + static_cast<uintptr_t>(pbytes);
}

struct Checked {
    tg_status status;
    bool noop;
};

Checked check_args(int64_t M, int64_t N, int64_t K, int dtype, const void *A, const void *B,
                   const void *bias, int epilogue, const void *C) {
    if (M < 0 || N < 0 || K < 0)
        return {TG_ERR_INVALID_ARG, false};
    if (dtype != TG_F16 && dtype != TG_BF16)
        return {TG_ERR_INVALID_ARG, false};
    if (epilogue != TG_EPI_NONE && epilogue != TG_EPI_BIAS && epilogue != TG_EPI_BIAS_GELU_TANH)
        return {TG_ERR_INVALID_ARG, false};
    if (epilogue == TG_EPI_NONE && bias != nullptr)
        return {TG_ERR_INVALID_ARG, false};
    if (M == 0 || N == 0)
        return {TG_OK, true};
    if (epilogue != TG_EPI_NONE && bias == nullptr)
        return {TG_ERR_INVALID_ARG, false};
    if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr)))
        return {TG_ERR_INVALID_ARG, false};
    const int64_t na = elements(M, K), nb = elements(K, N), nc = elements(M, N);
    const int64_t nbias = epilogue != TG_EPI_NONE ? N : 0;
    if (overlaps(C, 2 * (nc < 0 ? kMaxElements : nc), A, 2 * (na < 0 ? kMaxElements : na)) ||
        overlaps(C, 2 * (nc < 0 ? kMaxElements : nc), B, 2 * (nb < 0 ? kMaxElements : nb)) ||
        overlaps(C, 2 * (nc < 0 ? kMaxElements : nc), bias, 2 * nbias))
        return {TG_ERR_INVALID_ARG, false};
    if (na < 0 || nb < 0 || nc < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return {TG_ERR_UNSUPPORTED, false};
    return {TG_OK, false};
}

// The skinny kernel carries up to four 16-row blocks of A per workgroup.
constexpr int64_t kSkinnyMaxM = 64;
// Above 16 rows the skinny kernel beats the tiled family only while its
// 64-column slabs fit one round of workgroups (one per CU): measured on an
// MI355X at K = 4096 (A staged through LDS), M = 17..64 runs 1.5-2.0x faster
// than tiled for N = 4096 .. 16384 (N = 11008: M = 32 in 22.2 against 42.1
// us, M = 64 in 26.7 against 43.3 us; N = 16384: 26.3-30.1 against 43.0-45.0
// us), but 1.05-1.4x slower for N = 16388 .. 28672 (257-448 slabs: a second
// round of slabs).
constexpr int64_t kRowBlocksMaxN = 256 * 64;

bool skinny_ok(int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *bias, const void *C) {
    return M <= kSkinnyMaxM && K % 8 == 0 && N % 4 == 0 && aligned(A, 16) && aligned(B, 8) && aligned(C, 8) &&
           aligned(bias, 8);
}

// The tiled kernel addresses A and B through buffers that start 4 KiB before
// each operand and masks loads by adding 2^31 to their byte offsets, also for
// rows and k-rows of the padding past the operand's end; all such offsets
// must stay below 2^32, so each operand, padded to whole tiles, stays below
// 2 GiB less 64 KiB.  Any shape and any 2-byte alignment within that.
bool tiled_fits(int64_t M, int64_t N, int64_t K) {
    const int64_t limit = (int64_t(1) << 31) - 65536;
    return 2 * (M + 256) * K < limit && 2 * (K + 64) * (N + 256) < limit;
}

// The tiled kernel's instance without last-slice fix-ups and with 8-byte
// stores everywhere.
bool tiled_aligned(int64_t N, int64_t K, const void *A, const void *B, const void *bias, const void *C) {
    return K % 8 == 0 && N % 8 == 0 && aligned(A, 16) && aligned(B, 16) && aligned(C, 16) && aligned(bias, 8);
}

// Compute units of the device that `stream` belongs to (0 if unknown: the
// launchers then use one workgroup per tile).
constexpr int kMaxDevices = 64;
std::atomic<int> g_num_cu[kMaxDevices];

int num_cu_of(hipStream_t stream) {
    int dev = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 0;
    int n = g_num_cu[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return 0;
        g_num_cu[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Tile configuration for TG_TILES_AUTO: the one with the least predicted
// time.  The persistent grid runs the tiles in rounds of one (two for the
// 128 x 128 tiles) workgroup per CU; a round of one tile per CU on every CU
// takes a1 + b1 K, a round with two on some CUs a2 + b2 K, and a round on a
// fraction u of the CUs (1 - kappa (1 - u)) of the full-load time (less
// contention for caches and memory), with u taken as at least a quarter, the
// smallest fraction the sweep measures (a round on fewer CUs is not priced
// below it); rounds after the first take phi times
// longer, and misaligned shapes (K or N not a multiple of 8, or unaligned
// pointers) rho times longer.  The parameters come from a sweep of every
// configuration on one MI355X (bench.py --sweep: one tile per CU at two K,
// two per CU, a quarter of the CUs, the 8192-cube and a ragged shape); only
// their ratios between configurations matter.  A later configuration must
// beat the best earlier one by 2 % to be chosen, so that timing noise in the
// sweep does not decide between near-equal ones.
struct TileChoice {
    tg_tiles tiles;
    int bm, bn, occ;
    double a1, b1, a2, b2, kappa, phi, rho;
};
constexpr TileChoice kTileChoices[] = {
#include "tg_tile_model.inc"
};
constexpr int kDefaultCUs = 256;

double predicted_time(const TileChoice &c, int64_t M, int64_t N, int64_t K, int num_cu, bool aligned) {
    int64_t left = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const int64_t per_round = int64_t(num_cu) * c.occ;
    double t = 0.0;
    int rounds = 0;
    while (left > 0) {
        const int64_t busy = left < per_round ? left : per_round;
        if (busy > num_cu)
            t += c.a2 + c.b2 * double(K);
        else {
            const double u = double(busy) / double(num_cu);
            t += (c.a1 + c.b1 * double(K)) * (1.0 - c.kappa * (1.0 - (u > 0.25 ? u : 0.25)));
        }
        left -= busy;
        ++rounds;
    }
    if (rounds > 1)
        t *= c.phi;
    return aligned ? t : t * c.rho;
}

tg_tiles auto_tiles(int64_t M, int64_t N, int64_t K, int num_cu, bool aligned) {
    if (num_cu <= 0)
        num_cu = kDefaultCUs;
    tg_tiles pick = kTileChoices[0].tiles;
    double best = predicted_time(kTileChoices[0], M, N, K, num_cu, aligned);
    for (const TileChoice &c : kTileChoices) {
        const double t = predicted_time(c, M, N, K, num_cu, aligned);
        if (t < best * 0.98) {
            best = t;
            pick = c.tiles;
        }
    }
    return pick;
}

tg_path auto_path(int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *bias,
                  const void *C) {
    if (skinny_ok(M, N, K, A, B, bias, C) && (M <= 16 || N <= kRowBlocksMaxN))
        return TG_PATH_SKINNY;
    if (tiled_fits(M, N, K))
        return TG_PATH_TILED;
    return TG_PATH_TILED_GENERIC;
}

}  // namespace

TG_EXPORT tg_status tg_gemm_plan(int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void *A,
                                 const void *B, const void *bias, tg_epilogue epilogue, const void *C,
                                 tg_path *path_out) {
    if (path_out == nullptr)
        return TG_ERR_INVALID_ARG;
    const Checked c = check_args(M, N, K, dtype, A, B, bias, epilogue, C);
    if (c.status != TG_OK)
        return c.status;
    *path_out = c.noop ? TG_PATH_NONE : auto_path(M, N, K, A, B, bias, C);
    return TG_OK;
}

namespace {

// Split-K of the skinny kernel: the number of workgroups per 64-column slab
// for splits 0.  Splitting pays while the slabs alone leave CUs idle, and
// costs once the workgroups need a second round on the CUs (one workgroup
// fits a CU): measured on an MI355X, 64 slabs (N = 4096) run 1.8-2.6x faster
// with 4 splits, 16 slabs 2.4x with 8, while 172 slabs (N = 11008) run 20-50 %
// slower with any even split.  So the count is the largest that keeps
// slabs x splits within the CU count, and leaves each workgroup at least
// kMinSplitSteps 32-k steps.
constexpr int kMaxSplits = 64;
constexpr int kMinSplitSteps = 16;

int auto_splits(int64_t N, int64_t K, int num_cu) {
    if (num_cu <= 0)
        num_cu = kDefaultCUs;
    const int64_t slabs = (N + 63) / 64, steps = (K + 31) / 32;
    int64_t s = num_cu / slabs;
    s = s < steps / kMinSplitSteps ? s : steps / kMinSplitSteps;
    s = s < kMaxSplits ? s : kMaxSplits;
    return s > 1 ? static_cast<int>(s) : 1;
}

// Stream-K of the skinny kernel (TG_SPLIT_STREAM_K): the slabs x steps
// 32-k steps cut into equal contiguous ranges, one workgroup per CU, at
// least kMinSplitSteps steps each, at most kMaxStreamKGroups workgroups.
constexpr int kMaxStreamKGroups = 1024;

int streamk_groups(int64_t N, int64_t K, int num_cu) {
    if (num_cu <= 0)
        num_cu = kDefaultCUs;
    const int64_t total = ((N + 63) / 64) * ((K + 31) / 32);
    int64_t g = num_cu < kMaxStreamKGroups ? num_cu : kMaxStreamKGroups;
    g = g < total / kMinSplitSteps ? g : total / kMinSplitSteps;
    return g > 1 ? static_cast<int>(g) : 1;
}

// splits 0 on the skinny path: the even split above, or stream-K where it
// is predicted faster.  Cost in 32-k steps of the busiest CU, each step
// about 0.166 us on an MI355X whether 172 or 256 CUs stream: rounds of
// workgroups x steps per workgroup, plus the fixed cost of sharing slabs
// between workgroups, fitted to measured times of 16-row products (fp16,
// N = 4096, 11008, 16384, 19200, 28672; K = 512 .. 11008): about 7 us (42
// steps) for an even split (the partial stores, the counter round trip and
// the last workgroup's reads, one after the other at the end), about 12 us
// (71 steps) for stream-K (the same exchange, the loop through staged A
// slices, and workgroups streaming unrelated rows of B instead of the
// neighbouring slabs' same rows).  So stream-K pays only for long K where
// the slabs leave CUs idle (16 x 11008 x 11008: 47.5 against 55.0 us), not
// at the decode shape (16 x 11008 x 4096: 23.6 against 19.1 us).
constexpr int64_t kSplitFixedSteps = 42;
constexpr int64_t kStreamKFixedSteps = 71;

int auto_split_mode(int64_t N, int64_t K, int num_cu) {
    if (num_cu <= 0)
        num_cu = kDefaultCUs;
    const int64_t slabs = (N + 63) / 64, steps = (K + 31) / 32;
    const int s = auto_splits(N, K, num_cu);
    const int64_t rounds = (slabs * s + num_cu - 1) / num_cu;
    const int64_t even = rounds * ((steps + s - 1) / s) + (s > 1 ? kSplitFixedSteps : 0);
    const int g = streamk_groups(N, K, num_cu);
    const int64_t per = slabs * steps / g;   // the shorter ranges; the longer have one step more
    if (per < 1)
        return s;
    const int64_t parts = (steps + per - 1) / per + 1;   // the partial blocks a slab's last workgroup reads
    const int64_t sk = per + 1 + parts + kStreamKFixedSteps;
    return sk < even ? TG_SPLIT_STREAM_K : s;
}

// Workspace bytes of the skinny kernel's split mode (splits >= 1, or
// TG_SPLIT_STREAM_K with `groups` workgroups).
int64_t skinny_ws_bytes(int64_t slabs, int splits, int groups) {
    if (splits == TG_SPLIT_STREAM_K)
        return static_cast<int64_t>(tg::streamk_ws_bytes(slabs, groups));
    return static_cast<int64_t>(tg::split_ws_bytes(slabs, splits));
}

constexpr int kDefaultGroupM = 4;
constexpr int kMaxGroupM = 64;

tg_status run_gemm(tg_path path, tg_tiles tiles, int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void *A,
                   const void *B, const void *bias, tg_epilogue epilogue, void *C, void *stream,
                   int splits = 1, void *workspace = nullptr, int64_t workspace_bytes = 0, int group_m = 0) {
    if (path != TG_PATH_AUTO && path != TG_PATH_TILED && path != TG_PATH_TILED_GENERIC && path != TG_PATH_SKINNY)
        return TG_ERR_INVALID_ARG;
    if (tiles < TG_TILES_AUTO || tiles > tg::TILES_LAST)
        return TG_ERR_INVALID_ARG;
    if (group_m < 0 || group_m > kMaxGroupM)
        return TG_ERR_INVALID_ARG;
    const Checked c = check_args(M, N, K, dtype, A, B, bias, epilogue, C);
    if (c.status != TG_OK || c.noop)
        return c.status;
    if (path == TG_PATH_AUTO)
        path = auto_path(M, N, K, A, B, bias, C);
    else if ((path == TG_PATH_SKINNY && !skinny_ok(M, N, K, A, B, bias, C)) ||
             (path == TG_PATH_TILED && !tiled_fits(M, N, K)))
        return TG_ERR_UNSUPPORTED;

    tg::GemmArgs a;
    a.M = static_cast<int>(M);
    a.N = static_cast<int>(N);
    a.K = static_cast<int>(K);
    a.group_m = group_m > 0 ? group_m : kDefaultGroupM;
    a.A = static_cast<const uint16_t *>(A);
    a.B = static_cast<const uint16_t *>(B);
    a.bias = static_cast<const uint16_t *>(bias);
    a.C = static_cast<uint16_t *>(C);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (path == TG_PATH_SKINNY) {
        const int64_t slabs = (N + 63) / 64;
        if (M > 16)   // split-K is for a single row block; more rows run unsplit
            splits = 1;
        if (splits == 0)
            splits = auto_split_mode(N, K, num_cu_of(s));
        if (K == 0)   // nothing to divide
            splits = 1;
        const int groups = splits == TG_SPLIT_STREAM_K ? streamk_groups(N, K, num_cu_of(s)) : 0;
        if (splits > 1 || splits == TG_SPLIT_STREAM_K) {
            const int64_t need = skinny_ws_bytes(slabs, splits, groups);
            if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16))
                return TG_ERR_INVALID_ARG;
            const int64_t na = elements(M, K), nb = elements(K, N), nc = elements(M, N);
            if (overlaps(workspace, need, A, 2 * na) || overlaps(workspace, need, B, 2 * nb) ||
                overlaps(workspace, need, C, 2 * nc) || overlaps(workspace, need, bias, bias ? 2 * N : 0))
                return TG_ERR_INVALID_ARG;
        }
        e = tg::launch_skinny(dtype, epilogue, a,
                              groups > 0 ? tg::streamk_ws(workspace, slabs, groups) : tg::split_ws(workspace, slabs, splits),
                              s);
    } else if (path == TG_PATH_TILED) {
        const int cus = num_cu_of(s);
        const bool al = tiled_aligned(N, K, A, B, bias, C);
        if (tiles == TG_TILES_AUTO)
            tiles = auto_tiles(M, N, K, cus, al);
        e = tg::launch_tiled_vec(dtype, epilogue, a, al, tiles, cus, s);
    } else {
        e = tg::launch_tiled_generic(dtype, epilogue, a, s);
    }
    return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

}  // namespace

TG_EXPORT tg_status tg_gemm_path(tg_path path, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                                 const void *A, const void *B, const void *bias, tg_epilogue epilogue,
                                 void *C, void *stream) {
    return run_gemm(path, TG_TILES_AUTO, M, N, K, dtype, A, B, bias, epilogue, C, stream);
}

TG_EXPORT tg_status tg_gemm_tiled(tg_tiles tiles, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                                  const void *A, const void *B, const void *bias, tg_epilogue epilogue,
                                  void *C, void *stream) {
    return run_gemm(TG_PATH_TILED, tiles, M, N, K, dtype, A, B, bias, epilogue, C, stream);
}

TG_EXPORT tg_status tg_gemm_tiled_grouped(tg_tiles tiles, int group_m, int64_t M, int64_t N, int64_t K,
                                          tg_dtype dtype, const void *A, const void *B, const void *bias,
                                          tg_epilogue epilogue, void *C, void *stream) {
    if (group_m < 0 || group_m > kMaxGroupM)
        return TG_ERR_INVALID_ARG;
    return run_gemm(TG_PATH_TILED, tiles, M, N, K, dtype, A, B, bias, epilogue, C, stream, 1, nullptr, 0, group_m);
}

TG_EXPORT tg_status tg_gemm_tiles_plan(int64_t M, int64_t N, int64_t K, int num_cu, tg_tiles *tiles_out) {
    if (tiles_out == nullptr || M < 0 || N < 0 || K < 0)
        return TG_ERR_INVALID_ARG;
    *tiles_out = auto_tiles(M, N, K, num_cu, K % 8 == 0 && N % 8 == 0);
    return TG_OK;
}

TG_EXPORT tg_status tg_gemm(int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void *A, const void *B,
                            const void *bias, tg_epilogue epilogue, void *C, void *stream) {
    return tg_gemm_path(TG_PATH_AUTO, M, N, K, dtype, A, B, bias, epilogue, C, stream);
}

TG_EXPORT tg_status tg_gemm_split_plan(int64_t M, int64_t N, int64_t K, int num_cu, int *splits_out,
                                       int64_t *workspace_bytes_out) {
    if (splits_out == nullptr || workspace_bytes_out == nullptr || M < 0 || N < 0 || K < 0 || N > kMaxDim ||
        K > kMaxDim)
        return TG_ERR_INVALID_ARG;
    const int splits = (M <= 16 && M > 0 && N > 0 && K > 0) ? auto_split_mode(N, K, num_cu) : 1;
    *splits_out = splits;
    *workspace_bytes_out = skinny_ws_bytes((N + 63) / 64, splits, streamk_groups(N, K, num_cu));
    return TG_OK;
}

TG_EXPORT int64_t tg_gemm_split_workspace_bytes(int64_t N, int splits) {
    if (N < 0 || N > kMaxDim || splits < TG_SPLIT_STREAM_K || splits > kMaxSplits)
        return -1;
    return skinny_ws_bytes((N + 63) / 64, splits, kMaxStreamKGroups);
}

TG_EXPORT tg_status tg_gemm_split(int splits, int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void *A,
                                  const void *B, const void *bias, tg_epilogue epilogue, void *C, void *workspace,
                                  int64_t workspace_bytes, void *stream) {
    if (splits < TG_SPLIT_STREAM_K || splits > kMaxSplits || workspace_bytes < 0)
        return TG_ERR_INVALID_ARG;
    return run_gemm(TG_PATH_AUTO, TG_TILES_AUTO, M, N, K, dtype, A, B, bias, epilogue, C, stream, splits, workspace,
                    workspace_bytes);
}

namespace {

// Allocation-free split-K (tg_gemm_split_static): the workspace is a static
// device array, one copy per GPU, which the library holds until the process
// ends.  Its first kScratchCounterBytes hold the per-slab arrival counters,
// always at the same place, so that no call's partial sums ever land where
// another call expects zero counters; the partial blocks follow.  In host
// code `scratch` only names the host-side stand-in of the symbol: the device
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is used.
constexpr int64_t kScratchCounterBytes = tg::kSplitCounterBytes;   // 16384 slab counters, as in a workspace
constexpr int64_t kScratchPartialBytes = int64_t(4) << 20;    // 1024 partial blocks of 16 x 64 fp32
constexpr int64_t kScratchBytes = kScratchCounterBytes + kScratchPartialBytes;
static_assert(kScratchBytes == TG_SCRATCH_BYTES, "tg_gemm.h states the scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void zero_words_kernel(uint32_t *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0u;
}

std::mutex g_scratch_mutex;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the device of `stream`, set up on the
// first call for that device: symbol lookup with the device current, then a
// fill kernel on `stream` that zeroes the counters (every complete call
// leaves them zero again).  nullptr if the device is unknown or the lookup
// fails.
void *scratch_of(hipStream_t stream) {
    int dev = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr != nullptr)
        return ptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr != nullptr)
        return ptr;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess)
        return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess)
        return nullptr;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev)
        (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr)
        return nullptr;
    constexpr int words = static_cast<int>(kScratchCounterBytes / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3(words / 256), dim3(256), 0, stream, static_cast<uint32_t *>(p), words);
    if (hipGetLastError() != hipSuccess)
        return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace

TG_EXPORT tg_status tg_gemm_split_static(int splits, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                                         const void *A, const void *B, const void *bias, tg_epilogue epilogue,
                                         void *C, void *stream) {
    if (splits < TG_SPLIT_STREAM_K || splits > kMaxSplits)
        return TG_ERR_INVALID_ARG;
    const Checked c = check_args(M, N, K, dtype, A, B, bias, epilogue, C);
    if (c.status != TG_OK || c.noop)
        return c.status;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const tg_path path = auto_path(M, N, K, A, B, bias, C);
    if (path != TG_PATH_SKINNY || M > 16 || K == 0)   // no split, no workspace: exactly tg_gemm
        return run_gemm(TG_PATH_AUTO, TG_TILES_AUTO, M, N, K, dtype, A, B, bias, epilogue, C, stream);
    if (splits == 0)
        splits = auto_split_mode(N, K, num_cu_of(s));
    if (splits == 1)
        return run_gemm(TG_PATH_AUTO, TG_TILES_AUTO, M, N, K, dtype, A, B, bias, epilogue, C, stream);
    const int64_t slabs = (N + 63) / 64;
    const int groups = splits == TG_SPLIT_STREAM_K ? streamk_groups(N, K, num_cu_of(s)) : 0;
    const int64_t parts = groups > 0 ? groups + slabs - 1 : slabs * splits;
    if (slabs * 4 > kScratchCounterBytes || parts * 4096 > kScratchPartialBytes)
        return TG_ERR_UNSUPPORTED;
    char *ws = static_cast<char *>(scratch_of(s));
    if (ws == nullptr)
        return TG_ERR_LAUNCH;
    tg::GemmArgs a;
    a.M = static_cast<int>(M);
    a.N = static_cast<int>(N);
    a.K = static_cast<int>(K);
    a.group_m = kDefaultGroupM;
    a.A = static_cast<const uint16_t *>(A);
    a.B = static_cast<const uint16_t *>(B);
    a.bias = static_cast<const uint16_t *>(bias);
    a.C = static_cast<uint16_t *>(C);
    tg::SplitWs w;
    w.splits = groups > 0 ? 1 : splits;
    w.streamk = groups;
    w.count = reinterpret_cast<uint32_t *>(ws);
    w.part = reinterpret_cast<float *>(ws + kScratchCounterBytes);
    const hipError_t e = tg::launch_skinny(dtype, epilogue, a, w, s);
    return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

TG_EXPORT tg_status tg_elementwise(tg_elementwise_op op, int64_t M, int64_t N, tg_dtype dtype, const void *bias,
                                   const void *X, void *Y, void *stream) {
    if (M < 0 || N < 0)
        return TG_ERR_INVALID_ARG;
    if (dtype != TG_F16 && dtype != TG_BF16)
        return TG_ERR_INVALID_ARG;
    if (op != TG_EW_BIAS_ADD && op != TG_EW_GELU_TANH)
        return TG_ERR_INVALID_ARG;
    if ((op == TG_EW_BIAS_ADD) != (bias != nullptr))
        return TG_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return TG_OK;
    if (X == nullptr || Y == nullptr)
        return TG_ERR_INVALID_ARG;
    const int64_t n = elements(M, N);
    const int64_t ybytes = 2 * (n < 0 ? kMaxElements : n);
    if ((X != Y && overlaps(Y, ybytes, X, ybytes)) || overlaps(Y, ybytes, bias, 2 * N))
        return TG_ERR_INVALID_ARG;
    if (n < 0)
        return TG_ERR_UNSUPPORTED;
    const bool vec = N % 8 == 0 && aligned(X, 16) && aligned(Y, 16) && (bias == nullptr || aligned(bias, 16));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = tg::launch_elementwise(dtype, op, M, static_cast<int>(N), static_cast<const uint16_t *>(bias),
                                                static_cast<const uint16_t *>(X), static_cast<uint16_t *>(Y), vec,
                                                num_cu_of(s), s);
    return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

TG_EXPORT tg_status tg_gemm_unfused(int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void *A, const void *B,
                                    const void *bias, tg_epilogue epilogue, void *C, void *stream) {
    const Checked c = check_args(M, N, K, dtype, A, B, bias, epilogue, C);
    if (c.status != TG_OK || c.noop)
        return c.status;
    tg_status st = tg_gemm_path(TG_PATH_AUTO, M, N, K, dtype, A, B, nullptr, TG_EPI_NONE, C, stream);
    if (st == TG_OK && epilogue != TG_EPI_NONE)
        st = tg_elementwise(TG_EW_BIAS_ADD, M, N, dtype, bias, C, C, stream);
    if (st == TG_OK && epilogue == TG_EPI_BIAS_GELU_TANH)
        st = tg_elementwise(TG_EW_GELU_TANH, M, N, dtype, nullptr, C, C, stream);
    return st;
}

TG_EXPORT int64_t tg_w4_packed_bytes(int64_t K, int64_t N) {
    if (K < 0 || N < 0 || K % 32 != 0 || K > kMaxDim || N > kMaxDim)
        return -1;
    return 32 * K * ((N + 63) / 64);
}

TG_EXPORT tg_status tg_w4_pack(int64_t K, int64_t N, const void *q, void *packed, void *stream) {
    const int64_t bytes = tg_w4_packed_bytes(K, N);
    if (bytes < 0)
        return TG_ERR_INVALID_ARG;
    if (K == 0 || N == 0)
        return TG_OK;
    if (q == nullptr || packed == nullptr || !aligned(packed, 16))
        return TG_ERR_INVALID_ARG;
    if (overlaps(packed, bytes, q, K * N))
        return TG_ERR_INVALID_ARG;
    if (bytes > kMaxElements || elements(K, N) < 0)
        return TG_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = tg::launch_w4_pack(static_cast<int>(K), static_cast<int>(N),
                                            static_cast<const uint8_t *>(q), static_cast<uint8_t *>(packed), s);
    return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

namespace {

// Split-K of the 4-bit kernel, for splits 0: as for the skinny kernel, the
// largest count that keeps the workgroups (64-column slabs x 16-row blocks x
// splits) within one round on the CUs, with at least one scale group per
// wave (8 per workgroup).
int auto_w4_splits(int64_t M, int64_t N, int64_t K, int64_t group, int num_cu) {
    if (num_cu <= 0)
        num_cu = kDefaultCUs;
    const int64_t blocks = ((N + 63) / 64) * ((M + 15) / 16), groups = K / group;
    int64_t s = num_cu / blocks;
    s = s < groups / 8 ? s : groups / 8;
    s = s < kMaxSplits ? s : kMaxSplits;
    return s > 1 ? static_cast<int>(s) : 1;
}

tg_status run_w4(int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void *A, const void *packed,
                 const void *scales, int64_t group, const void *bias, tg_epilogue epilogue, void *C, void *stream,
                 int splits, void *workspace, int64_t workspace_bytes) {
    if (M < 0 || N < 0 || K < 0)
        return TG_ERR_INVALID_ARG;
    if (dtype != TG_F16 && dtype != TG_BF16)
        return TG_ERR_INVALID_ARG;
    if (epilogue != TG_EPI_NONE && epilogue != TG_EPI_BIAS && epilogue != TG_EPI_BIAS_GELU_TANH)
        return TG_ERR_INVALID_ARG;
    if (epilogue == TG_EPI_NONE && bias != nullptr)
        return TG_ERR_INVALID_ARG;
    if (group != 32 && group != 64 && group != 128 && group != 256)
        return TG_ERR_INVALID_ARG;
    if (K % group != 0)
        return TG_ERR_INVALID_ARG;
    if (M == 0 || N == 0)
        return TG_OK;
    if (epilogue != TG_EPI_NONE && bias == nullptr)
        return TG_ERR_INVALID_ARG;
    if (C == nullptr || (K > 0 && (A == nullptr || packed == nullptr || scales == nullptr)))
        return TG_ERR_INVALID_ARG;
    const int64_t na = elements(M, K), nc = elements(M, N), ns = elements(K / group, N);
    const int64_t pbytes = tg_w4_packed_bytes(K, N);
    const int64_t cb = 2 * (nc < 0 ? kMaxElements : nc);
    if (overlaps(C, cb, A, 2 * (na < 0 ? kMaxElements : na)) || overlaps(C, cb, packed, pbytes) ||
        overlaps(C, cb, scales, 2 * (ns < 0 ? kMaxElements : ns)) ||
        overlaps(C, cb, bias, epilogue != TG_EPI_NONE ? 2 * N : 0))
        return TG_ERR_INVALID_ARG;
    if (na < 0 || nc < 0 || ns < 0 || pbytes < 0 || pbytes > kMaxElements || M > 16 * 65535 || N > kMaxDim ||
        K > kMaxDim)
        return TG_ERR_UNSUPPORTED;
    tg::GemmArgs a;
    a.M = static_cast<int>(M);
    a.N = static_cast<int>(N);
    a.K = static_cast<int>(K);
    a.group_m = kDefaultGroupM;
    a.A = static_cast<const uint16_t *>(A);
    a.B = nullptr;
    a.bias = static_cast<const uint16_t *>(bias);
    a.C = static_cast<uint16_t *>(C);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t blocks = ((N + 63) / 64) * ((M + 15) / 16);
    if (splits == 0)
        splits = auto_w4_splits(M, N, K, group, num_cu_of(s));
    if (splits > 1) {
        const int64_t need = static_cast<int64_t>(tg::split_ws_bytes(blocks, splits));
        if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16))
            return TG_ERR_INVALID_ARG;
        if (overlaps(workspace, need, A, 2 * na) || overlaps(workspace, need, packed, pbytes) ||
            overlaps(workspace, need, scales, 2 * ns) || overlaps(workspace, need, C, 2 * nc) ||
            overlaps(workspace, need, bias, bias ? 2 * N : 0))
            return TG_ERR_INVALID_ARG;
    }
    const hipError_t e = tg::launch_w4(dtype, epilogue, a, static_cast<const uint8_t *>(packed),
                                       static_cast<const uint16_t *>(scales), static_cast<int>(group),
                                       tg::split_ws(workspace, blocks, splits), s);
    return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

}  // namespace

TG_EXPORT tg_status tg_gemm_w4(int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void *A, const void *packed,
                               const void *scales, int64_t group, const void *bias, tg_epilogue epilogue, void *C,
                               void *stream) {
    return run_w4(M, N, K, dtype, A, packed, scales, group, bias, epilogue, C, stream, 1, nullptr, 0);
}

TG_EXPORT tg_status tg_gemm_w4_split(int splits, int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void *A,
                                     const void *packed, const void *scales, int64_t group, const void *bias,
                                     tg_epilogue epilogue, void *C, void *workspace, int64_t workspace_bytes,
                                     void *stream) {
    if (splits < 0 || splits > kMaxSplits || workspace_bytes < 0)
        return TG_ERR_INVALID_ARG;
    return run_w4(M, N, K, dtype, A, packed, scales, group, bias, epilogue, C, stream, splits, workspace,
                  workspace_bytes);
}

TG_EXPORT int64_t tg_gemm_w4_split_workspace_bytes(int64_t M, int64_t N, int splits) {
    if (M < 0 || N < 0 || M > 16 * 65535 || N > kMaxDim || splits < 0 || splits > kMaxSplits)
        return -1;
    return static_cast<int64_t>(tg::split_ws_bytes(((N + 63) / 64) * ((M + 15) / 16), splits));
}

TG_EXPORT tg_status tg_gemm_w4_split_plan(int64_t M, int64_t N, int64_t K, int64_t group, int num_cu,
                                          int *splits_out, int64_t *workspace_bytes_out) {
    if (splits_out == nullptr || workspace_bytes_out == nullptr || M < 0 || N < 0 || K < 0 || M > 16 * 65535 ||
        N > kMaxDim || K > kMaxDim || (group != 32 && group != 64 && group != 128 && group != 256) ||
        K % group != 0)
        return TG_ERR_INVALID_ARG;
    const int splits = (M > 0 && N > 0) ? auto_w4_splits(M, N, K, group, num_cu) : 1;
    *splits_out = splits;
    *workspace_bytes_out = tg_gemm_w4_split_workspace_bytes(M, N, splits);
    return TG_OK;
}

TG_EXPORT tg_status tg_attention_fwd(int64_t batch, int64_t Sq, int64_t Sk, int64_t heads, int64_t head_dim,
                                     tg_dtype dtype, const void *Q, const void *K, const void *V, int causal,
                                     float scale, void *O, void *stream) {
    if (batch < 0 || Sq < 0 || Sk < 0 || heads < 0 || head_dim < 0)
        return TG_ERR_INVALID_ARG;
    if (dtype != TG_F16 && dtype != TG_BF16)
        return TG_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1)
        return TG_ERR_INVALID_ARG;
    if (causal && Sq != Sk)
        return TG_ERR_INVALID_ARG;
    if (!(scale >= 0.0f) || scale == HUGE_VALF)
        return TG_ERR_INVALID_ARG;
    if (batch == 0 || Sq == 0 || heads == 0 || head_dim == 0)
        return TG_OK;
    if (Q == nullptr || O == nullptr || (Sk > 0 && (K == nullptr || V == nullptr)))
        return TG_ERR_INVALID_ARG;
    // Sizes first (in double: the int64 products could overflow), then overlaps.
    const double limit = double((int64_t(1) << 31) - 65536);
    if (head_dim != 128 || heads > 65535 || batch > 65535 || double(batch) * double(heads) * double(Sq / 256 + 1) >= 2.0e9)
        return TG_ERR_UNSUPPORTED;
    if (2.0 * double(batch) * double(Sq + 256) * double(heads) * double(head_dim) >= limit ||
        2.0 * double(batch) * double(Sk + 64) * double(heads) * double(head_dim) >= limit)
        return TG_ERR_UNSUPPORTED;
    const int64_t q_bytes = 2 * batch * Sq * heads * head_dim;
    const int64_t kv_bytes = 2 * batch * Sk * heads * head_dim;
    if (overlaps(O, q_bytes, Q, q_bytes) || overlaps(O, q_bytes, K, kv_bytes) || overlaps(O, q_bytes, V, kv_bytes))
        return TG_ERR_INVALID_ARG;
    if (scale == 0.0f)
        scale = 1.0f / sqrtf((float)head_dim);
    tg::AttnArgs a;
    a.B = static_cast<int>(batch);
    a.Sq = static_cast<int>(Sq);
    a.Sk = static_cast<int>(Sk);
    a.H = static_cast<int>(heads);
    a.scale_log2 = scale * 1.4426950408889634f;
    a.causal = causal;
    a.Q = static_cast<const uint16_t *>(Q);
    a.K = static_cast<const uint16_t *>(K);
    a.V = static_cast<const uint16_t *>(V);
    a.O = static_cast<uint16_t *>(O);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = tg::launch_attention_fwd(dtype, a, s);
    return e == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

TG_EXPORT const char *tg_status_string(tg_status status) {
    switch (status) {
    case TG_OK: return "TG_OK";
    case TG_ERR_INVALID_ARG: return "TG_ERR_INVALID_ARG";
    case TG_ERR_UNSUPPORTED: return "TG_ERR_UNSUPPORTED";
    case TG_ERR_LAUNCH: return "TG_ERR_LAUNCH";
    }
    return "TG_UNKNOWN_STATUS";
}

TG_EXPORT const char *tg_version(void) { return "tg_gemm 0.1.0 gfx950"; }
