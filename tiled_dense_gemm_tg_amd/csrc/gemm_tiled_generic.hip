// gemm_tiled_generic.hip -- the 256 x 256 tiled MFMA GEMM for any shape and
// any alignment (gfx950).
//
// Same tiling as the vector kernel (gemm_tiled.hip) and the same fragment
// layout and epilogue, but operands are fetched element by element, so odd K
// or N and 2-byte-aligned pointers are fine.  Elements travel through
// registers: each thread gathers an 8 k x 8 m block of A and an 8 k x 8 n
// block of B per 64-wide k-slice, packs them, transposes B in registers with
// v_perm_b32 (both LDS tiles are K-contiguous, [row][64 k]) and writes them
// into the other of two LDS stages while the MFMAs run on the current one.
// Loads are range-checked buffer loads: k >= K reads as zero in both operands;
// rows past M and columns past N are never stored.
#include "tg_tile.h"

#include <type_traits>

namespace tg {
namespace {

using tile::BM;
using tile::BN;
using tile::NTHREADS;
using tile::OOB;
constexpr int BK = 64;
constexpr int CHUNKS = BK / 8;            // 16-byte chunks per LDS row
constexpr int TILE_U4 = BM * CHUNKS;      // 16-byte slots per operand per stage (32 KB)

// XOR swizzle of a row's 16-byte chunk: any 8 consecutive rows use 8
// different slots for one logical chunk, and any 16 consecutive rows split by
// parity into two sets of 8 different slots.
__device__ __forceinline__ int lds_slot(int row, int chunk) {
    return row * CHUNKS + (chunk ^ (((row >> 1) ^ (row << 2)) & 7));
}

// Thread t gathers A chunk c = t % 8 (8 k) of rows t/8 + 32 i (i = 0..7) and
// B rows 8 (t%8) + r (r = 0..7) of the 8 columns 8 (t/8) ...
struct Gather {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t a_row_off, a_row_step, b_col_off, b_row;
    int K, kq;

    __device__ __forceinline__ Gather(const GemmArgs &g, int m0, int n0, int tid) {
        ra = tile::buffer_of(g.A, 2u * (uint32_t)g.M * (uint32_t)g.K);
        rb = tile::buffer_of(g.B, 2u * (uint32_t)g.K * (uint32_t)g.N);
        K = g.K;
        kq = 8 * (tid & 7);
        a_row_off = 2u * ((uint32_t)(m0 + (tid >> 3)) * (uint32_t)g.K + (uint32_t)kq);
        a_row_step = 64u * (uint32_t)g.K;
        b_row = 2u * (uint32_t)g.N;
        b_col_off = (uint32_t)kq * b_row + 2u * (uint32_t)(n0 + 8 * (tid >> 3));
    }

    __device__ __forceinline__ void load(u32x4 (&xa)[8], u32x4 (&xb)[8], int k0) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint16_t e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t off =
                    (k0 + kq + q < K) ? a_row_off + (uint32_t)i * a_row_step + 2u * (uint32_t)(k0 + q) : OOB;
                e[q] = __builtin_amdgcn_raw_buffer_load_b16(ra, (int)off, 0, 0);
            }
            xa[i] = u32x4{pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7])};
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            uint16_t e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t off = (k0 + kq + r < K) ? b_col_off + (uint32_t)(k0 + r) * b_row + 2u * q : OOB;
                e[q] = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)off, 0, 0);
            }
            xb[r] = u32x4{pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7])};
        }
    }
};

__device__ __forceinline__ void store_a(u32x4 *__restrict__ As, const u32x4 (&xa)[8], int tid) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        As[lds_slot((tid >> 3) + 32 * i, c)] = xa[i];
}

// xb[r] holds B[k = 8g + r][n = 8c .. 8c+7]; column n = 8c + j becomes the
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

// Lane l reads chunk 2 s + l/32 (8 k) of rows 32 i + l%32 of A and of
// (B-transposed) rows 32 j + l%32, in its wave's quarter of the tile.
__device__ __forceinline__ void read_frag(u32x4 (&a)[4], u32x4 (&b)[4], const u32x4 *__restrict__ As,
                                          const u32x4 *__restrict__ Bs, int s, int wm, int wn, int lane) {
    const int lr = lane & 31;
    const int kc = 2 * s + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a[i] = As[lds_slot(wm * 128 + 32 * i + lr, kc)];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        b[j] = Bs[lds_slot(wn * 128 + 32 * j + lr, kc)];
}

template <class T, int EPI>
__global__ __launch_bounds__(NTHREADS) void gemm_tiled_generic_kernel(GemmArgs args) {
    __shared__ u32x4 smem[4 * TILE_U4];  // A stage 0, A stage 1, B stage 0, B stage 1
    int tm, tn;
    tile::tile_of_workgroup(args.M, args.N, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const Gather ld(args, m0, n0, tid);
    auto A_st = [&](int st) { return smem + st * TILE_U4; };
    auto B_st = [&](int st) { return smem + (2 + st) * TILE_U4; };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x16{};

    // Slice t lives in stage t&1; its successor is gathered into registers
    // during slice t and written to the other stage before the barrier.
    const int nk = (args.K + BK - 1) / BK;
    u32x4 xa[8], xb[8];
    if (nk > 0) {
        ld.load(xa, xb, 0);
        store_a(A_st(0), xa, tid);
        store_b(B_st(0), xb, tid);
    }
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
        const int cur = t & 1;
        const bool more = t + 1 < nk;
        if (more)
            ld.load(xa, xb, (t + 1) * BK);
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            u32x4 a[4], b[4];
            read_frag(a, b, A_st(cur), B_st(cur), s, wm, wn, lane);
            tile::mfma_step<T>(a, b, acc);
        }
        if (more) {
            store_a(A_st(cur ^ 1), xa, tid);
            store_b(B_st(cur ^ 1), xb, tid);
        }
        __syncthreads();
    }
    tile::store_tile<T, EPI, false>(args, acc, m0, n0, wm, wn, lane);
}

template <class T, int EPI>
hipError_t launch_typed(const GemmArgs &a, hipStream_t stream) {
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    hipLaunchKernelGGL((gemm_tiled_generic_kernel<T, EPI>), dim3(tiles), dim3(NTHREADS), 0, stream, a);
    return hipGetLastError();
}

template <class T>
hipError_t launch_epi(int epi, const GemmArgs &a, hipStream_t stream) {
    switch (epi) {
    case EPI_NONE: return launch_typed<T, EPI_NONE>(a, stream);
    case EPI_BIAS: return launch_typed<T, EPI_BIAS>(a, stream);
    default: return launch_typed<T, EPI_BIAS_GELU_TANH>(a, stream);
    }
}

}  // namespace

hipError_t launch_tiled_generic(int dtype, int epi, const GemmArgs &a, hipStream_t stream) {
    return dtype == 0 ? launch_epi<F16>(epi, a, stream) : launch_epi<BF16>(epi, a, stream);
}

}  // namespace tg
