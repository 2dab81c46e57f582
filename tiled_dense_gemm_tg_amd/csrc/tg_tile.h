// tg_tile.h -- pieces shared by the tiled GEMM kernels: the XCD-aware tile
// raster (any tile size), buffer descriptors, and for the register-gathered
// 256 x 256 kernel the MFMA step and the fused epilogue + store of a wave's
// 128 x 128 quarter of the C tile.
#pragma once

#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace tile {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int NTHREADS = 256;             // 4 wave64s, each owning 128 x 128 of C
constexpr int GROUP_M = 4;                // tile rows per raster group unless the caller picks another
constexpr int NUM_XCD = 8;
constexpr uint32_t OOB = 0xFFFFFFF0u;     // byte offset beyond every operand (< 2^32 - 32 bytes)

// Workgroups are dispatched round-robin over the 8 XCDs, so tile id w runs
// on XCD x = w % 8 (also for a persistent grid whose size is a multiple of
// 8) as the (w / 8)-th tile there.  Give each XCD a contiguous range of
// logical tiles (the first total % 8 XCDs one more than the others: XCD x
// runs exactly that many ids), and walk them group_m tile-rows at a time,
// column by column, so that the tiles running together on one XCD share A
// row-panels and B column-panels in that XCD's L2.  A bijection on
// [0, tiles_m * tiles_n), for any tile size and count and group_m >= 1.
__device__ __forceinline__ void tile_of_index(int tiles_m, int tiles_n, int w, int group_m, int &tm, int &tn) {
    const int total = tiles_m * tiles_n;
    {
        const int q = total / NUM_XCD, r = total % NUM_XCD;
        const int x = w % NUM_XCD;
        w = x * q + min(x, r) + w / NUM_XCD;
    }
    const int per_group = group_m * tiles_n;
    const int grp = w / per_group;
    const int first_m = grp * group_m;
    const int rows = min(tiles_m - first_m, group_m);
    const int rem = w - grp * per_group;
    tm = first_m + rem % rows;
    tn = rem / rows;
}

// The raster of 256 x 256 tiles over an M x N output.
__device__ __forceinline__ void tile_of_workgroup(int M, int N, int w, int &tm, int &tn) {
    tile_of_index((M + BM - 1) / BM, (N + BN - 1) / BN, w, GROUP_M, tm, tn);
}

// Raw buffer (stride 0) over [base, base + bytes): loads beyond the range
// return zero and stores beyond it are dropped.  0x00020000 is the gfx9-family
// word 3 (32-bit data format) of the buffer resource.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 MFMAs of one k-step.  a[i] holds rows 32 i + l%32 of A (8 k each),
// b[j] columns 32 j + l%32 of B; the B fragment goes first, so
// acc[i][j] = D with D[n][m] = sum_k B[k][n] A[m][k].
template <class T>
__device__ __forceinline__ void mfma_step(const u32x4 (&a)[4], const u32x4 (&b)[4], f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = T::mfma32(b[j], a[i], acc[i][j]);
}

// How store_tile writes C: element by element (any shape and alignment);
// 8-byte groups of four columns (N % 4 == 0, C and bias 8-byte aligned); or
// 8-byte groups wherever a group lies inside the row and elements elsewhere
// (any N and 2-byte alignment: the hardware takes unaligned 8-byte accesses,
// but a group that crossed the row end would write into the next row).
enum StoreMode { STORE_ELEM = 0, STORE_VEC = 1, STORE_GROUP = 2 };

// Fused epilogue and store.  Lane l of wave (wm, wn) holds, in acc[i][j][e],
// C[m][n] with m = m0 + wm*128 + 32 i + l%32 and
// n = n0 + wn*128 + 32 j + 8 (e/4) + 4 (l/32) + e%4: four consecutive columns
// per (i, j, e/4).
template <class T, int EPI, int MODE>
__device__ __forceinline__ void store_tile(const GemmArgs &args, const f32x16 (&acc)[4][4], int m0, int n0, int wm,
                                           int wn, int lane) {
    const int M = args.M, N = args.N;
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
                if constexpr (MODE == STORE_VEC) {
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
                const u32x2 packed = u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
                if constexpr (MODE == STORE_VEC) {
                    const uint32_t off = (m < M && n < N) ? base : OOB;
                    __builtin_amdgcn_raw_buffer_store_b64(packed, rc, (int)off, 0, 0);
                } else if constexpr (MODE == STORE_GROUP) {
                    if (n + 3 < N) {
                        const uint32_t off = m < M ? base : OOB;
                        __builtin_amdgcn_raw_buffer_store_b64(packed, rc, (int)off, 0, 0);
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const uint32_t off = (m < M && n + r < N) ? base + 2u * r : OOB;
                            __builtin_amdgcn_raw_buffer_store_b16(o[r], rc, (int)off, 0, 0);
                        }
                    }
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

}  // namespace tile
}  // namespace tg
