// gemm_tiled_generic.hip -- the 256 x 256 tiled MFMA GEMM for any shape and
// any alignment (gfx950), for operands beyond the direct-load kernel's size
// limit (2 GiB per padded operand), up to 2^31 - 64 elements.
//
// Same tiling as the vector kernel (gemm_tiled.hip) and the same fragment
// layout and epilogue, but rows of A and B may start at any 2-byte boundary
// (odd K or N, 2-byte-aligned pointers), so operands cannot go straight to
// LDS as aligned 16-byte pieces.  Each 8-element chunk is fetched as a
// dword-aligned 16-byte load plus one dword and shifted into place, through
// registers: each thread gathers an 8 k x 8 m block of A and an 8 k x 8 n
// block of B per 64-wide k-slice, transposes B in registers with v_perm_b32
// (both LDS tiles are K-contiguous, [row][64 k]) and writes them into the
// other of two LDS stages while the MFMAs run on the current one.  Stores are
// element-granular.  Loads are range-checked buffer loads.
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

// Out-of-range byte offset for these loads: it and offset + 16 both stay
// beyond every operand (operands are below 2^32 - 32 bytes).
constexpr uint32_t OOB_G = 0xFFFFFFE0u;

// Buffer over [p, p + bytes) whose base is rounded down to 4 bytes, so that
// every dword-aligned offset is a dword-aligned address; `adj` (0 or 2) is
// added to all offsets.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dword_buffer(const void *p, uint32_t bytes, uint32_t &adj) {
    adj = (uint32_t)((uintptr_t)p & 2u);
    return tile::buffer_of((const char *)p - adj, bytes + adj);
}

// One chunk = 8 consecutive 16-bit elements at byte offset `ob` (2-byte
// aligned) of a buffer of `limit` bytes, fetched as the 16 bytes at the
// enclosing dword-aligned offset o4 plus the next dword, shifted down by
// sh = 0 or 2 bytes (v_alignbyte_b32).  A 16-byte load that crosses the end of
// the buffer reads as all zeros, so a chunk whose bytes straddle the end
// (only the last chunks of an operand) is fetched element by element instead.
// The loads of all chunks are issued before any result is used, so they are
// all in flight together: issue() for every chunk, then fix() (the rare
// straddling chunks), then value().
struct Chunk {
    u32x4 d;
    uint32_t e;
    uint32_t ob, sh;
    bool straddle;

    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t limit) {
        ob = off;
        const uint32_t o4 = off & ~3u;
        sh = off & 2u;
        straddle = o4 < limit && o4 + 16u + 2u * sh > limit;
        // straddling chunks skip the vector loads (offset pushed out of
        // range); the empty asm keeps the choice an OR instead of a branch
        uint32_t m = straddle ? OOB_G : 0u;
        asm volatile("" : "+v"(m));
        d = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(o4 | m), 0, 0);
        e = __builtin_amdgcn_raw_buffer_load_b32(r, (int)((o4 + 16u) | m), 0, 0);
    }

    __device__ __forceinline__ void fix(__amdgpu_buffer_rsrc_t r) {
        if (straddle) {
            uint16_t v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                v[q] = __builtin_amdgcn_raw_buffer_load_b16(r, (int)(ob + 2u * q), 0, 0);
            d = u32x4{pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
            e = 0u;
            sh = 0u;
        }
    }

    __device__ __forceinline__ u32x4 value() const {
        return u32x4{__builtin_amdgcn_alignbyte(d.y, d.x, sh), __builtin_amdgcn_alignbyte(d.z, d.y, sh),
                     __builtin_amdgcn_alignbyte(d.w, d.z, sh), __builtin_amdgcn_alignbyte(e, d.w, sh)};
    }
};

// Thread t gathers A chunk c = t % 8 (8 k) of rows t/8 + 32 i (i = 0..7) and
// B rows 8 (t%8) + r (r = 0..7) of the 8 columns 8 (t/8) ...  Elements k >= K
// are zeroed in both operands (A per element, B per row); rows past M and
// columns past N only reach outputs that are never stored.
struct Gather {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t a_row_off, a_row_step, b_col_off, b_row;
    uint32_t a_limit, b_limit;   // buffer sizes in bytes
    int K, kq;

    __device__ __forceinline__ Gather(const GemmArgs &g, int m0, int n0, int tid) {
        uint32_t a_adj, b_adj;
        ra = dword_buffer(g.A, 2u * (uint32_t)g.M * (uint32_t)g.K, a_adj);
        rb = dword_buffer(g.B, 2u * (uint32_t)g.K * (uint32_t)g.N, b_adj);
        a_limit = a_adj + 2u * (uint32_t)g.M * (uint32_t)g.K;
        b_limit = b_adj + 2u * (uint32_t)g.K * (uint32_t)g.N;
        K = g.K;
        kq = 8 * (tid & 7);
        a_row_off = a_adj + 2u * ((uint32_t)(m0 + (tid >> 3)) * (uint32_t)g.K + (uint32_t)kq);
        a_row_step = 64u * (uint32_t)g.K;
        b_row = 2u * (uint32_t)g.N;
        b_col_off = b_adj + (uint32_t)kq * b_row + 2u * (uint32_t)(n0 + 8 * (tid >> 3));
    }

    __device__ __forceinline__ void load(u32x4 (&xa)[8], u32x4 (&xb)[8], int k0) const {
        // number of this thread's 8 A elements with k < K (same for all rows)
        const int nv = K - (k0 + kq);
        Chunk ca[8], cb[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t off = (nv > 0) ? a_row_off + (uint32_t)i * a_row_step + 2u * (uint32_t)k0 : OOB_G;
            ca[i].issue(ra, off, a_limit);
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const uint32_t off = (k0 + kq + r < K) ? b_col_off + (uint32_t)(k0 + r) * b_row : OOB_G;
            cb[r].issue(rb, off, b_limit);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            ca[i].fix(ra);
#pragma unroll
        for (int r = 0; r < 8; ++r)
            cb[r].fix(rb);
        u32x4 amask;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            amask[i] = (2 * i + 1 < nv) ? 0xFFFFFFFFu : ((2 * i < nv) ? 0x0000FFFFu : 0u);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            xa[i] = ca[i].value() & amask;
#pragma unroll
        for (int r = 0; r < 8; ++r)
            xb[r] = cb[r].value();
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
    tile::tile_of_workgroup(args.M, args.N, blockIdx.x, tm, tn);
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
    tile::store_tile<T, EPI, tile::STORE_ELEM>(args, acc, m0, n0, wm, wn, lane);
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
