// gemm_skinny.hip -- the M <= 64 (decode-shaped) GEMM for gfx950.
//
// With at most 16 rows of A the product does 2*M flops per B element, far
// below what keeps MFMA busy, so the kernel is shaped by HBM: B is read from
// memory exactly once, in 8-byte pieces that coalesce into 128-byte row
// segments, with many loads in flight per lane.  The first TileLang page
// ("TileLang: writing LLM GPU kernels by thinking in tiles", section 2,
// "A back-of-the-envelope calculation") frames the same point: what costs is
// moving each value, not the arithmetic.
//
// Layout of the work:
//   * one workgroup per 64-column slab of B and C; its 4 waves (one per
//     SIMD, so a lane may hold up to 512 registers) split the K
//     range into contiguous parts and each streams its part of the slab;
//   * per 32-k step a lane loads rows kb + 8 h + r (r = 0..7, h = lane/16) of
//     the four columns 4 p .. 4 p + 3 (p = lane % 16) and transposes them in
//     registers (v_perm_b32) into four 8-k column vectors;
//   * v_mfma_f32_16x16x32 takes those vectors as its 16-row operand (row p of
//     MFMA j is column 4 p + j) and the 16 x 32 slice of A (8 k of row p per
//     lane, one 16-byte load from L2) as its 16-column operand, so the 16
//     MFMA columns are the (at most 16) rows of A;
//   * loads come in batches of 2 steps, double-buffered in registers, so the
//     next batch is in flight while the current one is multiplied; where
//     every wave has 17 to 32 steps (K = 4096: 32) a wave first copies its
//     whole slice of A into its own 32 KB of LDS by direct loads of 4 rows x
//     256 contiguous bytes and reads it into registers in the MFMA layout,
//     so that its loop streams only B;
//   * 17 <= M <= 64: two to four such 16-row blocks of A per workgroup,
//     each with its own MFMAs on the same transposed B vectors, so B is
//     still read once (A then comes from L2 in every step; no preload);
//   * the 4 waves' fp32 partial sums are added in LDS in a fixed order (no
//     atomics, so results are reproducible), then the fused epilogue and
//     8-byte stores;
//   * split-K (splits > 1, a grid of slabs x splits): when there are too few
//     slabs to fill the chip, each slab's K range is also divided over
//     `splits` workgroups, which pass their partial slabs through a
//     workspace; the last to arrive adds them in split order and finishes.
// Loads are range-checked buffer loads; k >= K reads zero in both operands.
#include "tg_device.h"
#include "tg_launch.h"
#include "tg_direct.h"
#include "tg_split.h"

namespace tg {
namespace {

constexpr int SLAB = 64;       // columns per workgroup
constexpr int WAVES = 4;       // waves per workgroup (one per SIMD), splitting K
constexpr int UNROLL = 2;      // 32-k steps per load batch (two batches in flight)
constexpr int NTHREADS = 64 * WAVES;
constexpr int PRE = 32;        // most 32-k steps per wave whose A slice is preloaded into registers
constexpr uint32_t OOB = 0xFFFFFFF0u;    // byte offset beyond every operand
constexpr uint32_t ASHIFT = 4096;        // the staged-A buffer starts this far before A
// Cache policy of the B loads: non-temporal.  Each B element is read once,
// so its lines need not displace the A rows every workgroup re-reads from
// L2 (16x4096x11008: 20.35 -> 19.8 us per launch).
constexpr int CPOL_NT = 2;

using namespace direct;

template <int RB>
struct ABatch {
    u32x4 v[UNROLL][RB];
};
__device__ __forceinline__ ABatch<1> u32x4_pair(u32x4 a, u32x4 b) { return ABatch<1>{{{a}, {b}}}; }

// RB: 16-row blocks of A (and C) per workgroup, 1..4 (M <= 16 RB).  Every
// block multiplies the same B vectors, so B is still read once; the preload
// path and split-K are for RB = 1 only.  One wave per SIMD gives a lane up
// to 512 registers: four blocks need more than the 256 of two waves per
// SIMD (with 8 waves they spilled and ran 2-3x slower than three blocks),
// and every instance ran as fast or faster on 4 waves than on 8 (M = 16,
// K = 4096 with the preload: 18.95 against 19.86 us).
template <class T, int EPI, bool PRELOAD, int RB>
__global__ __launch_bounds__(NTHREADS) void gemm_skinny_kernel(GemmArgs args, SplitWs ws) {
    static_assert(RB >= 1 && RB <= 4 && (RB == 1 || !PRELOAD), "row blocks");
    // Per wave RS floats of LDS: 32 KB with the preload (its slice of A,
    // 16 rows x 32 PRE k), else 16 KB; after its k-loop, its RB 16 x 64 fp32
    // partial sums (4 KB each).  Each wave touches only its own region until
    // the barrier before the cross-wave reduction.
    constexpr int RS = PRELOAD ? 256 * PRE : 4096;
    __shared__ __attribute__((aligned(16))) u32x4 smem[WAVES * RS / 4];
    auto red = [&](int w, int b, int i, int l) __attribute__((always_inline)) -> float & {
        return reinterpret_cast<float *>(smem)[RS * w + 1024 * b + 64 * i + l];
    };
    const int M = args.M, N = args.N, K = args.K;
    const uint16_t *__restrict__ A = args.A;
    const uint16_t *__restrict__ B = args.B;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: loop control stays scalar
    const int p = lane & 15;
    const int h = lane >> 4;
    const int nb = blockIdx.x * SLAB;
    const int ncol = nb + 4 * p;              // N % 4 == 0: all four columns valid or none

    // this workgroup's part of the 32-k steps (all of them without split-K),
    // divided over its waves
    const int steps = (K + 31) / 32;
    const int splits = ws.splits;
    const int split = blockIdx.y;
    const int sp_begin = (int)(((int64_t)steps * split) / splits);
    const int sp_len = (int)(((int64_t)steps * (split + 1)) / splits) - sp_begin;
    const int s_begin = sp_begin + (int)(((int64_t)sp_len * wave) / WAVES);
    const int s_end = sp_begin + (int)(((int64_t)sp_len * (wave + 1)) / WAVES);

    f32x4 acc[RB][4];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[b][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Batches of UNROLL 32-k steps, double-buffered in registers: the loads
    // of the next batch are in flight while the current one is multiplied.
    // Range-checked buffer loads (out of range reads zero): k >= K and steps
    // past this wave's range read zero in both operands; rows m >= M and
    // columns n >= N only reach outputs that are never stored.
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(A), (short)0,
                                                                        (int)(2u * (uint32_t)M * (uint32_t)K),
                                                                        0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(B), (short)0,
                                                                        (int)(2u * (uint32_t)K * (uint32_t)N),
                                                                        0x00020000);
    const uint32_t a_row = 2u * (uint32_t)p * (uint32_t)K;   // row p of block 0; block b is 16 b rows further
    const uint32_t a_blk = 32u * (uint32_t)K;
    const uint32_t b_col = 2u * (uint32_t)ncol;
    const uint32_t b_row = 2u * (uint32_t)N;
    // Offsets of masked loads are OR-ed with OOB; the mask goes through an
    // empty asm so the compiler keeps the OR instead of turning the choice
    // into a branch around each load.
    auto mask_of = [&](bool ok) __attribute__((always_inline)) {
        uint32_t m = ok ? 0u : OOB;
        asm volatile("" : "+v"(m));
        return m;
    };
    auto load_batch = [&](u32x2 (&vb)[UNROLL][8], ABatch<RB> &va, int s0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kb = (s0 + u) * 32 + 8 * h;
            // K % 8 == 0, so rows kb .. kb + 7 (and the A chunk's 8 k) are
            // all inside [0, K) or all outside.
            const uint32_t mk = mask_of(s0 + u < s_end && kb < K);
#pragma unroll
            for (int b = 0; b < RB; ++b)
                va.v[u][b] = __builtin_amdgcn_raw_buffer_load_b128(
                    ra, (int)((a_row + (uint32_t)b * a_blk + 2u * (uint32_t)kb) | mk), 0, 0);
            const uint32_t boff = (uint32_t)kb * b_row + b_col;
#pragma unroll
            for (int r = 0; r < 8; ++r)
                vb[u][r] = __builtin_amdgcn_raw_buffer_load_b64(rb, (int)((boff + (uint32_t)r * b_row) | mk), 0, CPOL_NT);
        }
    };
    auto mma_batch = [&](const u32x2 (&vb)[UNROLL][8], const ABatch<RB> &va) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d = j >> 1;
                u32x4 w;
                if (j & 1) {
                    w.x = perm_hi(vb[u][0][d], vb[u][1][d]);
                    w.y = perm_hi(vb[u][2][d], vb[u][3][d]);
                    w.z = perm_hi(vb[u][4][d], vb[u][5][d]);
                    w.w = perm_hi(vb[u][6][d], vb[u][7][d]);
                } else {
                    w.x = perm_lo(vb[u][0][d], vb[u][1][d]);
                    w.y = perm_lo(vb[u][2][d], vb[u][3][d]);
                    w.z = perm_lo(vb[u][4][d], vb[u][5][d]);
                    w.w = perm_lo(vb[u][6][d], vb[u][7][d]);
                }
#pragma unroll
                for (int b = 0; b < RB; ++b)
                    acc[b][j] = T::mfma16(w, va.v[u][b], acc[b][j]);
            }
        }
    };
    // Every batch's loads are issued before the previous batch is
    // multiplied (sched_barrier keeps that order); loads past the wave's
    // range are masked, read nothing and give zeros.
    u32x2 vb0[UNROLL][8], vb1[UNROLL][8];
    ABatch<RB> va0, va1;
    if constexpr (PRELOAD) {
        // Every wave has PRE / 2 < steps <= PRE (K = 4096 on 4 waves: 32;
        // the host picks this instance only then) and reads its whole slice
        // of A (16 rows x 32 PRE k) into registers first, so the loop
        // streams only B.  A separate instance rather than a branch: merged
        // with the other loop, the compiler's wait counts would stall on
        // loads of the path not taken.
        // The slice goes through the wave's LDS region: PRE direct loads,
        // each of 4 rows x 256 contiguous bytes (half the cache lines of
        // 16 rows x 64 bytes), then 16-byte reads in the MFMA layout.
        // Load j = 4 c4 + rq: row r = 4 rq + lane / 16 and k = 32 s_begin +
        // 128 c4 + 8 c, where the lane's 16-byte slot lane % 16 of the row
        // holds logical chunk c = slot ^ r (the swizzle that makes the reads
        // of 16 rows' same chunk hit 16 different bank groups).  LDS byte
        // 4096 c4 + 256 r + 16 slot of the region.  Chunks at k >= K or past
        // the wave's steps, and rows >= M, are out of range and read zero.
        const uint32_t region = lds_address(smem) + 4u * RS * (uint32_t)wave;
        auto load_b = [&](u32x2 (&vb)[UNROLL][8], int s0) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int kb = (s0 + u) * 32 + 8 * h;
                const uint32_t mk = mask_of(s0 + u < s_end && kb < K);
                const uint32_t boff = (uint32_t)kb * b_row + b_col;
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    vb[u][r] = __builtin_amdgcn_raw_buffer_load_b64(rb, (int)((boff + (uint32_t)r * b_row) | mk), 0,
                                                                    CPOL_NT);
            }
        };
        // B's first two batches go out around the A loads, so that the wait
        // for A below leaves a full batch of B in flight (waiting for A
        // before issuing the second batch cost 1.7 us per launch)
        load_b(vb0, s_begin);
        {
            const i32x4 rs = rsrc_words((const char *)A - ASHIFT, 2u * (uint32_t)M * (uint32_t)K + ASHIFT);
            const int r0 = lane >> 4;
            const int slot = lane & 15;
            const int kend = min(K, 32 * s_end);   // k past the wave's range reads zero too
#pragma unroll
            for (int c4 = 0; c4 < PRE / 4; ++c4) {
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int r = 4 * rq + r0;
                    const int k = 32 * s_begin + 128 * c4 + 8 * (slot ^ r);
                    const uint32_t off = (ASHIFT - 1024u * (uint32_t)rq + 2u * ((uint32_t)r * (uint32_t)K + (uint32_t)k)) +
                                         (k < kend ? 0u : 0x80000000u);
                    dma16_rq(rq, rs, off, region + 4096u * (uint32_t)c4);
                }
            }
        }
        load_b(vb1, s_begin + UNROLL);
        // the PRE A loads are older than the second batch's 8 UNROLL B loads
        wait_vmcnt<8 * UNROLL>();
        u32x4 pa[PRE];
#pragma unroll
        for (int i = 0; i < PRE; ++i) {
            const uint32_t c = (uint32_t)((4 * (i & 3) + h) ^ p);
            pa[i] = *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)(region + 4096u * (uint32_t)(i >> 2) +
                                                                                 256u * (uint32_t)p + 16u * c);
        }
#pragma unroll
        for (int bi = 0; bi < PRE / UNROLL; bi += 2) {
            if (bi > 0)
                load_b(vb1, s_begin + (bi + 1) * UNROLL);
            __builtin_amdgcn_sched_barrier(0);
            mma_batch(vb0, u32x4_pair(pa[bi * UNROLL], pa[bi * UNROLL + 1]));
            __builtin_amdgcn_sched_barrier(0);
            if (bi + 2 < PRE / UNROLL)
                load_b(vb0, s_begin + (bi + 2) * UNROLL);
            __builtin_amdgcn_sched_barrier(0);
            mma_batch(vb1, u32x4_pair(pa[(bi + 1) * UNROLL], pa[(bi + 1) * UNROLL + 1]));
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        load_batch(vb0, va0, s_begin);
        for (int s0 = s_begin; s0 < s_end; s0 += 2 * UNROLL) {
            load_batch(vb1, va1, s0 + UNROLL);
            __builtin_amdgcn_sched_barrier(0);
            mma_batch(vb0, va0);
            __builtin_amdgcn_sched_barrier(0);
            if (s0 + UNROLL >= s_end)
                break;
            load_batch(vb0, va0, s0 + 2 * UNROLL);
            __builtin_amdgcn_sched_barrier(0);
            mma_batch(vb1, va1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // acc[b][j][e] is D_j[row 4 h + e][col p] of row block b:
    // C[m = 16 b + p][n = nb + 16 h + 4 e + j].
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                red(wave, b, 4 * e + j, lane) = acc[b][j][e];
    __syncthreads();

    // the sum over the waves of (row block b, column group e) for every lane
    auto wave_sum = [&](int b, int e, float (&y)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w)
                s += red(w, b, 4 * e + j, lane);
            y[j] = s;
        }
    };
    uint16_t *__restrict__ C = args.C;
    auto finish = [&](int b, int e, const float (&y)[4]) __attribute__((always_inline)) {
        const int m = 16 * b + p;
        const int n = nb + 16 * h + 4 * e;
        if (m >= M || n >= N)
            return;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (EPI != EPI_NONE) {
            const u32x2 raw = *reinterpret_cast<const u32x2 *>(args.bias + n);
            bv[0] = T::to_f32((uint16_t)(raw.x & 0xffff));
            bv[1] = T::to_f32((uint16_t)(raw.x >> 16));
            bv[2] = T::to_f32((uint16_t)(raw.y & 0xffff));
            bv[3] = T::to_f32((uint16_t)(raw.y >> 16));
        }
        uint16_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = T::from_f32(epilogue<EPI>(y[j], bv[j]));
        *reinterpret_cast<u32x2 *>(C + (uint32_t)m * (uint32_t)N + n) = u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
    };
    if constexpr (RB == 1) {
        // waves 0..3 each finish one of the four column groups e of every lane
        const int e = wave & 3;
        float y[4] = {0.f, 0.f, 0.f, 0.f};
        if (wave < 4)
            wave_sum(0, e, y);
        if (splits > 1 && !split_exchange(ws, blockIdx.x, split, y, e))
            return;
        if (wave < 4)
            finish(0, e, y);
    } else {
        // the 4 RB (row block, column group) pairs are spread over the waves
#pragma unroll
        for (int q0 = 0; q0 < 4 * RB; q0 += WAVES) {
            const int q = q0 + wave;
            if (q < 4 * RB) {
                float y[4];
                wave_sum(q >> 2, q & 3, y);
                finish(q >> 2, q & 3, y);
            }
        }
    }
}

template <class T, int EPI, int RB>
hipError_t launch_rows(const GemmArgs &a, const SplitWs &ws, hipStream_t stream) {
    const int slabs = (a.N + SLAB - 1) / SLAB;
    hipLaunchKernelGGL((gemm_skinny_kernel<T, EPI, false, RB>), dim3(slabs, ws.splits), dim3(NTHREADS), 0, stream, a,
                       ws);
    return hipGetLastError();
}

template <class T, int EPI>
hipError_t launch_typed(const GemmArgs &a, const SplitWs &ws, hipStream_t stream) {
    const int slabs = (a.N + SLAB - 1) / SLAB;
    if (a.M > 16) {   // several row blocks: no split-K (the host passes splits = 1)
        if (ws.splits != 1 || a.M > 64)
            return hipErrorInvalidValue;
        if (a.M > 48)
            return launch_rows<T, EPI, 4>(a, ws, stream);
        return a.M <= 32 ? launch_rows<T, EPI, 2>(a, ws, stream) : launch_rows<T, EPI, 3>(a, ws, stream);
    }
    // every wave's share of the 32-k steps is floor or ceil of a split's
    // share / WAVES, and a split's share floor or ceil of steps / splits
    const int64_t steps = (a.K + 31) / 32;
    const int64_t lo = steps / ws.splits, hi = (steps + ws.splits - 1) / ws.splits;
    if (lo / WAVES > PRE / 2 && (hi + WAVES - 1) / WAVES <= PRE)
        hipLaunchKernelGGL((gemm_skinny_kernel<T, EPI, true, 1>), dim3(slabs, ws.splits), dim3(NTHREADS), 0, stream, a,
                           ws);
    else
        return launch_rows<T, EPI, 1>(a, ws, stream);
    return hipGetLastError();
}

template <class T>
hipError_t launch_epi(int epi, const GemmArgs &a, const SplitWs &ws, hipStream_t stream) {
    switch (epi) {
    case EPI_NONE: return launch_typed<T, EPI_NONE>(a, ws, stream);
    case EPI_BIAS: return launch_typed<T, EPI_BIAS>(a, ws, stream);
    default: return launch_typed<T, EPI_BIAS_GELU_TANH>(a, ws, stream);
    }
}

}  // namespace

hipError_t launch_skinny(int dtype, int epi, const GemmArgs &a, const SplitWs &ws, hipStream_t stream) {
    return dtype == 0 ? launch_epi<F16>(epi, a, ws, stream) : launch_epi<BF16>(epi, a, ws, stream);
}

}  // namespace tg
