// gemm_tiled.hip -- tiled MFMA GEMM for gfx950 (MI355X).
//
// The tiling is the one the TileLang pages teach ("TileLang: writing LLM GPU
// kernels by thinking in tiles", section 2 and the section 3 listing; "TileLang:
// you write the dataflow, the compiler owns the schedule", sections "The tile
// program" and "What a tile costs, exactly"): one workgroup per output tile,
// a loop over k-slices that copies an A tile and a B tile from global memory
// into on-chip memory, a tile matrix multiply into a register accumulator
// held in fp32, and one write-back of the tile after the loop; the copy of
// slice k+1 overlaps the multiply of slice k.  The sizes and mechanics are
// chosen for CDNA4 rather than taken from the pages' NVIDIA example:
//
//   * tile 256 x 256 x 64, 256 threads = 4 wave64s, each wave owning a
//     128 x 128 quarter of C as 4 x 4 v_mfma_f32_32x32x16 accumulators
//     (256 fp32 values per lane, held in AGPR/VGPR);
//   * two LDS stages of 2 x 32 KB (128 KB of the 160 KB LDS), one barrier per
//     k-slice; global loads for slice t+1 are issued before the MFMAs of
//     slice t and written to the other stage after them;
//   * both operands are stored in LDS K-contiguous ([row][64 k]), because a
//     16-bit MFMA takes eight consecutive k of one row (A) or one column (B)
//     per lane.  A arrives that way; B (row-major K x N) is transposed in
//     registers on its way into LDS: each thread loads an 8 k x 8 n block
//     with eight 16-byte loads and rebuilds it as 8 n x 8 k with v_perm_b32;
//   * a 16-byte-chunk XOR swizzle within each 128-byte LDS row (see swz);
//   * the MFMA is issued with the B fragment as its first operand, so each
//     lane ends up with 4 consecutive output columns of one row, stored as a
//     single 8-byte write after the fused epilogue;
//   * workgroups are remapped so that each XCD (8 on MI355X, dispatched
//     round-robin) works on a contiguous, grouped block of tiles, which keeps
//     the A and B panels those tiles share inside that XCD's L2.
//
// Edge tiles (M, N, K not multiples of the tile) are masked: elements outside
// the matrices are loaded as zeros in both A and B, and stores are skipped.
#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int NTHREADS = 256;
constexpr int CHUNKS = BK / 8;            // 16-byte chunks per LDS row
constexpr int TILE_U4 = BM * CHUNKS;      // 16-byte slots per operand per stage (32 KB)
constexpr int GROUP_M = 4;                // tile rows per raster group
constexpr int NUM_XCD = 8;
static_assert(BM == BN, "A and B tiles share one LDS layout");

// XOR swizzle of a row's 16-byte chunk index.  A fragment read takes one
// logical chunk from 32 consecutive rows.  f(row) permutes the 8 chunk slots
// so that any 8 consecutive rows (one 128-byte pass over 32 four-byte banks)
// use 8 different slots, and any 16 consecutive rows split by parity into
// two sets of 8 different slots (one 256-byte pass over 64 banks covers two
// 128-byte rows).
__device__ __forceinline__ int swz(int row, int chunk) {
    return chunk ^ (((row >> 1) ^ (row << 2)) & 7);
}
__device__ __forceinline__ int lds_slot(int row, int chunk) {
    return row * CHUNKS + swz(row, chunk);
}

__device__ __forceinline__ void tile_of_workgroup(int M, int N, int &tm, int &tn) {
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int total = tiles_m * tiles_n;
    int w = blockIdx.x;
    if (total % NUM_XCD == 0)
        w = (w % NUM_XCD) * (total / NUM_XCD) + w / NUM_XCD;
    const int per_group = GROUP_M * tiles_n;
    const int grp = w / per_group;
    const int first_m = grp * GROUP_M;
    const int rows = min(tiles_m - first_m, GROUP_M);
    const int rem = w - grp * per_group;
    tm = first_m + rem % rows;
    tn = rem / rows;
}

// ---- global -> registers ------------------------------------------------
// A tile (BM x BK): thread t loads chunk c = t % 8 (8 k) of rows t/8 + 32 i.
template <bool VEC>
__device__ __forceinline__ void load_a(u32x4 (&ra)[8], const uint16_t *__restrict__ A, int M, int K,
                                       int m0, int k0, int tid) {
    const int c = tid & 7;
    const int gk = k0 + 8 * c;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int gm = m0 + (tid >> 3) + 32 * i;
        const uint16_t *p = A + (uint32_t)gm * (uint32_t)K + gk;
        if constexpr (VEC) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (gm < M && gk < K)
                v = *reinterpret_cast<const u32x4 *>(p);
            ra[i] = v;
        } else {
            uint16_t e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                e[q] = (gm < M && gk + q < K) ? p[q] : (uint16_t)0;
            ra[i] = u32x4{pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7])};
        }
    }
}

// B tile (BK x BN): thread t loads rows k0 + 8 g + r (g = t % 8, r = 0..7) of
// n-chunk c = t / 8 (8 n), i.e. an 8 x 8 block.
template <bool VEC>
__device__ __forceinline__ void load_b(u32x4 (&rb)[8], const uint16_t *__restrict__ B, int N, int K,
                                       int n0, int k0, int tid) {
    const int g = tid & 7;
    const int gn = n0 + 8 * (tid >> 3);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int gk = k0 + 8 * g + r;
        const uint16_t *p = B + (uint32_t)gk * (uint32_t)N + gn;
        if constexpr (VEC) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (gk < K && gn < N)
                v = *reinterpret_cast<const u32x4 *>(p);
            rb[r] = v;
        } else {
            uint16_t e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                e[q] = (gk < K && gn + q < N) ? p[q] : (uint16_t)0;
            rb[r] = u32x4{pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7])};
        }
    }
}

// ---- registers -> LDS ---------------------------------------------------
__device__ __forceinline__ void store_a(u32x4 *__restrict__ As, const u32x4 (&ra)[8], int tid) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        As[lds_slot((tid >> 3) + 32 * i, c)] = ra[i];
}

// rb[r] holds B[k = 8g + r][n = 8c .. 8c+7]; write column n = 8c + j as the
// 8 consecutive k of LDS row n, chunk g.
__device__ __forceinline__ void store_b(u32x4 *__restrict__ Bs, const u32x4 (&rb)[8], int tid) {
    const int g = tid & 7;
    const int c = tid >> 3;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int d = j >> 1;
        u32x4 w;
        if (j & 1) {
            w.x = perm_hi(rb[0][d], rb[1][d]);
            w.y = perm_hi(rb[2][d], rb[3][d]);
            w.z = perm_hi(rb[4][d], rb[5][d]);
            w.w = perm_hi(rb[6][d], rb[7][d]);
        } else {
            w.x = perm_lo(rb[0][d], rb[1][d]);
            w.y = perm_lo(rb[2][d], rb[3][d]);
            w.z = perm_lo(rb[4][d], rb[5][d]);
            w.w = perm_lo(rb[6][d], rb[7][d]);
        }
        Bs[lds_slot(8 * c + j, g)] = w;
    }
}

// ---- LDS -> MFMA --------------------------------------------------------
// Wave (wm, wn) owns rows wm*128.. and columns wn*128.. of the tile.  For the
// k-step s (16 k), lane l reads the chunk 2 s + l/32 of row 32 i + l%32 of
// A and of row (column of B) 32 j + l%32.  acc[i][j] = D with
// D[n][m] = sum_k B[k][n] A[m][k]: lane l holds m = l%32 and
// n = 8 (e/4) + 4 (l/32) + e%4 for its 16 values e.
template <class T>
__device__ __forceinline__ void mma_stage(const u32x4 *__restrict__ As, const u32x4 *__restrict__ Bs,
                                          f32x16 (&acc)[4][4], int wm, int wn, int lane) {
    const int lr = lane & 31;
    const int lh = lane >> 5;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
        const int kc = 2 * s + lh;
        u32x4 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = As[lds_slot(wm * 128 + 32 * i + lr, kc)];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            b[j] = Bs[lds_slot(wn * 128 + 32 * j + lr, kc)];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = T::mfma32(b[j], a[i], acc[i][j]);
    }
}

template <class T, int EPI, bool VEC>
__global__ __launch_bounds__(NTHREADS) void gemm_tiled_kernel(GemmArgs args) {
    __shared__ u32x4 smem[4 * TILE_U4];  // A stage 0, A stage 1, B stage 0, B stage 1
    const int M = args.M, N = args.N, K = args.K;
    const uint16_t *__restrict__ A = args.A;
    const uint16_t *__restrict__ B = args.B;

    int tm, tn;
    tile_of_workgroup(M, N, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x16{};

    const int nk = (K + BK - 1) / BK;
    u32x4 ra[8], rb[8];
    if (nk > 0) {
        load_a<VEC>(ra, A, M, K, m0, 0, tid);
        load_b<VEC>(rb, B, N, K, n0, 0, tid);
        store_a(smem, ra, tid);
        store_b(smem + 2 * TILE_U4, rb, tid);
    }
    __syncthreads();

    for (int t = 0; t < nk; ++t) {
        const int cur = t & 1;
        const bool more = t + 1 < nk;
        if (more) {
            load_a<VEC>(ra, A, M, K, m0, (t + 1) * BK, tid);
            load_b<VEC>(rb, B, N, K, n0, (t + 1) * BK, tid);
        }
        mma_stage<T>(smem + cur * TILE_U4, smem + (2 + cur) * TILE_U4, acc, wm, wn, lane);
        if (more) {
            store_a(smem + (cur ^ 1) * TILE_U4, ra, tid);
            store_b(smem + (2 + (cur ^ 1)) * TILE_U4, rb, tid);
        }
        __syncthreads();
    }

    // ---- fused epilogue and store ------------------------------------------
    const int lr = lane & 31;
    const int lh = lane >> 5;
    uint16_t *__restrict__ C = args.C;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn * 128 + 32 * j + 8 * q + 4 * lh;
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (EPI != EPI_NONE) {
                if constexpr (VEC) {
                    if (n < N) {
                        const u32x2 raw = *reinterpret_cast<const u32x2 *>(args.bias + n);
                        bv[0] = T::to_f32((uint16_t)(raw.x & 0xffff));
                        bv[1] = T::to_f32((uint16_t)(raw.x >> 16));
                        bv[2] = T::to_f32((uint16_t)(raw.y & 0xffff));
                        bv[3] = T::to_f32((uint16_t)(raw.y >> 16));
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N)
                            bv[r] = T::to_f32(args.bias[n + r]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + wm * 128 + 32 * i + lr;
                uint16_t o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[r] = T::from_f32(epilogue<EPI>(acc[i][j][4 * q + r], bv[r]));
                if (m < M) {
                    uint16_t *p = C + (uint32_t)m * (uint32_t)N + n;
                    if constexpr (VEC) {
                        if (n < N)
                            *reinterpret_cast<u32x2 *>(p) = u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (n + r < N)
                                p[r] = o[r];
                    }
                }
            }
        }
    }
}

template <class T, int EPI>
hipError_t launch_typed(bool vec, const GemmArgs &a, hipStream_t stream) {
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (vec)
        hipLaunchKernelGGL((gemm_tiled_kernel<T, EPI, true>), dim3(tiles), dim3(NTHREADS), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_tiled_kernel<T, EPI, false>), dim3(tiles), dim3(NTHREADS), 0, stream, a);
    return hipGetLastError();
}

template <class T>
hipError_t launch_epi(int epi, bool vec, const GemmArgs &a, hipStream_t stream) {
    switch (epi) {
    case EPI_NONE: return launch_typed<T, EPI_NONE>(vec, a, stream);
    case EPI_BIAS: return launch_typed<T, EPI_BIAS>(vec, a, stream);
    default: return launch_typed<T, EPI_BIAS_GELU_TANH>(vec, a, stream);
    }
}

}  // namespace

hipError_t launch_tiled(int dtype, int epi, bool vec, const GemmArgs &a, hipStream_t stream) {
    return dtype == 0 ? launch_epi<F16>(epi, vec, a, stream) : launch_epi<BF16>(epi, vec, a, stream);
}

}  // namespace tg
