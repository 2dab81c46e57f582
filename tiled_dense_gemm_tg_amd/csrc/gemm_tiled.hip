// gemm_tiled.hip -- tiled MFMA GEMM for gfx950 (MI355X).
//
// The tiling is the one the TileLang pages teach ("TileLang: writing LLM GPU
// kernels by thinking in tiles", section 2 and the section 3 listing; "TileLang:
// you write the dataflow, the compiler owns the schedule", sections "The tile
// program", "What a tile costs, exactly" and "Software pipelining"): one
// workgroup per output tile, a loop over k-slices that copies an A tile and a B
// tile from global memory into on-chip memory, a tile matrix multiply into a
// register accumulator held in fp32, and one write-back of the tile after the
// loop, with the copies of later slices overlapping the multiply of the
// current one.  The sizes and mechanics are chosen for CDNA4 rather than taken
// from the pages' NVIDIA example:
//
//   * tile 256 x 256 x 64, 256 threads = 4 wave64s, each wave owning a
//     128 x 128 quarter of C as 4 x 4 v_mfma_f32_32x32x16 accumulators
//     (256 fp32 values per lane, held in AGPRs);
//   * two LDS stages of 2 x 32 KB (128 KB of the 160 KB LDS) and one barrier per
//     k-slice; a slice's global loads are issued two k-steps before the end of
//     the previous slice and written to LDS one k-step into the current one, so
//     a full slice of MFMA work hides their latency;
//   * both operands are stored in LDS K-contiguous ([row][64 k]), because a
//     16-bit MFMA takes eight consecutive k of one row (A) or one column (B)
//     per lane.  A arrives that way; B (row-major K x N) is transposed in
//     registers on its way into LDS: each thread loads an 8 k x 8 n block
//     with eight 16-byte loads and rebuilds it as 8 n x 8 k with v_perm_b32;
//   * a 16-byte-chunk XOR swizzle within each 128-byte LDS row (see swz);
//   * MFMA fragments are double-buffered in registers: the reads for k-step
//     s+1 are issued between the MFMAs of step s, and instruction-group hints
//     interleave the LDS writes and global loads with the MFMAs too, so the
//     matrix unit is fed from one wave per SIMD without waiting on LDS;
//   * the MFMA is issued with the B fragment as its first operand, so each
//     lane ends up with 4 consecutive output columns of one row, stored as a
//     single 8-byte write after the fused epilogue;
//   * workgroups are remapped so that each XCD (8 on MI355X, dispatched
//     round-robin) works on a contiguous, grouped block of tiles, which keeps
//     the A and B panels those tiles share inside that XCD's L2.
//
// Global loads are raw buffer loads over each operand's exact byte range: the
// hardware returns zero for offsets beyond the range, so edge tiles need no
// branches and no access can leave the operand.  k >= K is forced out of range
// in both A and B (the K tail must be zero on both sides); rows m >= M and
// columns n >= N are never stored, so what they load does not matter.
#include "tg_device.h"
#include "tg_launch.h"

#include <type_traits>

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
constexpr uint32_t OOB = 0xFFFFFFF0u;     // byte offset beyond every operand (< 2^32 - 32 bytes)
// Added to an offset below 2^31 it lands beyond any operand of the vector
// path, whose operands are limited to 2^31 bytes; an additive bump (rather
// than a select) keeps the compiler from turning the mask into a branch.
constexpr uint32_t OOB_BUMP = 0x80000000u;
static_assert(BM == BN, "A and B tiles share one LDS layout");

// sched_group_barrier masks
constexpr int SG_VALU = 0x002;
constexpr int SG_MFMA = 0x008;
constexpr int SG_VMEM_READ = 0x020;
constexpr int SG_DS_READ = 0x100;
constexpr int SG_DS_WRITE = 0x200;

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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void *base, uint32_t bytes) {
    // raw buffer (stride 0), range checked against `bytes`; 0x00020000 is the
    // gfx9-family word 3 (32-bit data format) of the buffer resource
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// ---- global -> registers ------------------------------------------------
// Thread t: A chunk c = t % 8 (8 k) of rows t/8 + 32 i (i = 0..7);
//           B rows 8 g + r (g = t % 8, r = 0..7) of the 8 columns 8 (t/8)...
struct Loader {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t a_row_off;   // byte offset of (m0 + t/8, 8 (t%8)) in A
    uint32_t a_row_step;  // bytes between rows i and i+1 (32 rows of A)
    uint32_t b_col_off;   // byte offset of (8 (t%8), n0 + 8 (t/8)) in B
    uint32_t b_row;       // bytes per row of B
    int K;
    int ak;               // first k of this thread's A chunk, relative to k0
    int bk;               // first k of this thread's B rows, relative to k0

    __device__ __forceinline__ Loader(const GemmArgs &g, int m0, int n0, int tid) {
        ra = buffer_of(g.A, 2u * (uint32_t)g.M * (uint32_t)g.K);
        rb = buffer_of(g.B, 2u * (uint32_t)g.K * (uint32_t)g.N);
        K = g.K;
        ak = 8 * (tid & 7);
        bk = 8 * (tid & 7);
        a_row_off = 2u * ((uint32_t)(m0 + (tid >> 3)) * (uint32_t)g.K + (uint32_t)ak);
        a_row_step = 64u * (uint32_t)g.K;
        b_row = 2u * (uint32_t)g.N;
        b_col_off = (uint32_t)bk * b_row + 2u * (uint32_t)(n0 + 8 * (tid >> 3));
    }

    // 16-byte loads (K % 8 == 0, N % 8 == 0, 16-byte aligned operands)
    __device__ __forceinline__ void load_vec(u32x4 (&xa)[8], u32x4 (&xb)[8], int k0) const {
        const uint32_t a_bump = (k0 + ak < K) ? 0u : OOB_BUMP;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t off = a_row_off + (uint32_t)i * a_row_step + 2u * (uint32_t)k0 + a_bump;
            xa[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const uint32_t bump = (k0 + bk + r < K) ? 0u : OOB_BUMP;
            const uint32_t off = b_col_off + (uint32_t)(k0 + r) * b_row + bump;
            xb[r] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)off, 0, 0);
        }
    }

    // element loads (any shape, any alignment); the k >= K mask is applied per
    // element, rows and columns past the edges are handled as for load_vec
    __device__ __forceinline__ void load_elem(u32x4 (&xa)[8], u32x4 (&xb)[8], int k0) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint16_t e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const bool ok = k0 + ak + q < K;
                const uint32_t off = ok ? a_row_off + (uint32_t)i * a_row_step + 2u * (uint32_t)(k0 + q) : OOB;
                e[q] = __builtin_amdgcn_raw_buffer_load_b16(ra, (int)off, 0, 0);
            }
            xa[i] = u32x4{pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7])};
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            uint16_t e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const bool ok = k0 + bk + r < K;
                const uint32_t off = ok ? b_col_off + (uint32_t)(k0 + r) * b_row + 2u * q : OOB;
                e[q] = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)off, 0, 0);
            }
            xb[r] = u32x4{pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7])};
        }
    }
};

// ---- registers -> LDS ---------------------------------------------------
__device__ __forceinline__ void store_a(u32x4 *__restrict__ As, const u32x4 (&xa)[8], int tid) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        As[lds_slot((tid >> 3) + 32 * i, c)] = xa[i];
}

// xb[r] holds B[k = 8g + r][n = 8c .. 8c+7]; write column n = 8c + j as the
// 8 consecutive k of LDS row n, chunk g.
__device__ __forceinline__ void store_b(u32x4 *__restrict__ Bs, const u32x4 (&xb)[8], int tid) {
    const int g = tid & 7;
    const int c = tid >> 3;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int d = j >> 1;
        u32x4 w;
        if (j & 1) {
            w.x = perm_hi(xb[0][d], xb[1][d]);
            w.y = perm_hi(xb[2][d], xb[3][d]);
            w.z = perm_hi(xb[4][d], xb[5][d]);
            w.w = perm_hi(xb[6][d], xb[7][d]);
        } else {
            w.x = perm_lo(xb[0][d], xb[1][d]);
            w.y = perm_lo(xb[2][d], xb[3][d]);
            w.z = perm_lo(xb[4][d], xb[5][d]);
            w.w = perm_lo(xb[6][d], xb[7][d]);
        }
        Bs[lds_slot(8 * c + j, g)] = w;
    }
}

// ---- LDS -> MFMA --------------------------------------------------------
// Wave (wm, wn) owns rows wm*128.. and columns wn*128.. of the tile.  For
// k-step s (16 k), lane l reads chunk 2 s + l/32 of row 32 i + l%32 of A and
// of row (column of B) 32 j + l%32.
struct Frag {
    u32x4 a[4], b[4];
};

__device__ __forceinline__ void read_frag(Frag &f, const u32x4 *__restrict__ As, const u32x4 *__restrict__ Bs,
                                          int s, int wm, int wn, int lane) {
    const int lr = lane & 31;
    const int kc = 2 * s + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        f.a[i] = As[lds_slot(wm * 128 + 32 * i + lr, kc)];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        f.b[j] = Bs[lds_slot(wn * 128 + 32 * j + lr, kc)];
}

// acc[i][j] = D with D[n][m] = sum_k B[k][n] A[m][k]: lane l holds m = l%32
// and n = 8 (e/4) + 4 (l/32) + e%4 for its 16 values e.
template <class T>
__device__ __forceinline__ void mfma_step(const Frag &f, f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = T::mfma32(f.b[j], f.a[i], acc[i][j]);
}

// Ordering hints for one k-step of 16 MFMAs: the 8 fragment reads of the
// next step go one after each of the first 8 MFMAs, then (VALU, EXTRA) groups
// of the other work of the step go after the MFMAs, first the 8 second-half
// MFMAs and, with FIRST_HALF, also after the first 8.
template <int EXTRA_MASK, int EXTRA_PER_MFMA, int VALU_PER_MFMA, bool FIRST_HALF>
__device__ __forceinline__ void interleave_hint() {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
        if constexpr (FIRST_HALF && EXTRA_PER_MFMA > 0)
            __builtin_amdgcn_sched_group_barrier(EXTRA_MASK, EXTRA_PER_MFMA, 0);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        if constexpr (VALU_PER_MFMA > 0)
            __builtin_amdgcn_sched_group_barrier(SG_VALU, VALU_PER_MFMA, 0);
        if constexpr (EXTRA_PER_MFMA > 0)
            __builtin_amdgcn_sched_group_barrier(EXTRA_MASK, EXTRA_PER_MFMA, 0);
    }
}

template <class T, int EPI, bool VEC>
__global__ __launch_bounds__(NTHREADS) void gemm_tiled_kernel(GemmArgs args) {
    __shared__ u32x4 smem[4 * TILE_U4];  // A stage 0, A stage 1, B stage 0, B stage 1
    const int M = args.M, N = args.N, K = args.K;

    int tm, tn;
    tile_of_workgroup(M, N, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;

    const Loader ld(args, m0, n0, tid);
    auto load = [&](u32x4 (&xa)[8], u32x4 (&xb)[8], int kt) __attribute__((always_inline)) {
        if constexpr (VEC)
            ld.load_vec(xa, xb, kt * BK);
        else
            ld.load_elem(xa, xb, kt * BK);
    };
    auto A_st = [&](int st) { return smem + st * TILE_U4; };
    auto B_st = [&](int st) { return smem + (2 + st) * TILE_U4; };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x16{};

    const int nk = (K + BK - 1) / BK;
    u32x4 xa[8], xb[8];
    Frag f0, f1;
    if (nk > 0) {
        load(xa, xb, 0);
        store_a(A_st(0), xa, tid);
        store_b(B_st(0), xb, tid);
        if (nk > 1)
            load(xa, xb, 1);
        __syncthreads();
        read_frag(f0, A_st(0), B_st(0), 0, wm, wn, lane);
    }

    // One k-slice t in LDS stage t&1, its fragments for step 0 already in f0
    // and slice t+1 already in xa/xb:
    //   step 0: MFMA f0 | read step 1 -> f1
    //   step 1: MFMA f1 | read step 2 -> f0 | write xa/xb (slice t+1) to the other stage
    //   step 2: MFMA f0 | read step 3 -> f1 | issue global loads of slice t+2
    //   barrier (slice t+1 complete in LDS, all reads of slice t done)
    //   step 3: MFMA f1 | read step 0 of slice t+1 -> f0
    // The other stage was last read in slice t-1, before the previous barrier.
    auto slice = [&](int t, auto store_next, auto load_next2, auto read_next) __attribute__((always_inline)) {
        const int cur = t & 1;
        const u32x4 *As = A_st(cur);
        const u32x4 *Bs = B_st(cur);

        read_frag(f1, As, Bs, 1, wm, wn, lane);
        mfma_step<T>(f0, acc);
        if constexpr (VEC)
            interleave_hint<0, 0, 0, false>();
        __builtin_amdgcn_sched_barrier(0);

        read_frag(f0, As, Bs, 2, wm, wn, lane);
        if constexpr (decltype(store_next)::value) {
            store_a(A_st(cur ^ 1), xa, tid);
            store_b(B_st(cur ^ 1), xb, tid);
        }
        mfma_step<T>(f1, acc);
        if constexpr (VEC)
            interleave_hint<SG_DS_WRITE, 1, 4, true>();
        __builtin_amdgcn_sched_barrier(0);

        read_frag(f1, As, Bs, 3, wm, wn, lane);
        if constexpr (decltype(load_next2)::value)
            load(xa, xb, t + 2);
        mfma_step<T>(f0, acc);
        if constexpr (VEC)
            interleave_hint<SG_VMEM_READ, 2, 2, false>();
        __syncthreads();

        if constexpr (decltype(read_next)::value)
            read_frag(f0, A_st(cur ^ 1), B_st(cur ^ 1), 0, wm, wn, lane);
        mfma_step<T>(f1, acc);
        if constexpr (VEC)
            interleave_hint<0, 0, 0, false>();
        __builtin_amdgcn_sched_barrier(0);
    };

    using yes = std::true_type;
    using no = std::false_type;
    int t = 0;
    for (; t + 2 < nk; ++t)
        slice(t, yes{}, yes{}, yes{});
    if (t + 1 < nk) {
        slice(t, yes{}, no{}, yes{});
        ++t;
    }
    if (t < nk)
        slice(t, no{}, no{}, no{});

    // ---- fused epilogue and store ------------------------------------------
    const int lr = lane & 31;
    const int lh = lane >> 5;
    const __amdgpu_buffer_rsrc_t rc = buffer_of(args.C, 2u * (uint32_t)M * (uint32_t)N);
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
                const uint32_t base = 2u * ((uint32_t)m * (uint32_t)N + (uint32_t)n);
                if constexpr (VEC) {
                    const uint32_t off = (m < M && n < N) ? base : OOB;
                    __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])}, rc,
                                                          (int)off, 0, 0);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t off = (m < M && n + r < N) ? base + 2u * r : OOB;
                        __builtin_amdgcn_raw_buffer_store_b16(o[r], rc, (int)off, 0, 0);
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
