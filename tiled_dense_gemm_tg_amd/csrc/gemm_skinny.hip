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
//     so that its loop streams only B; with more steps, the slice goes
//     through the same 32 KB in chunks, read from LDS step by step;
//   * 17 <= M <= 64: two to four such 16-row blocks of A per workgroup,
//     each with its own MFMAs on the same transposed B vectors, so B is
//     still read once; their slices of A are staged in chunks the same way;
//   * the 4 waves' fp32 partial sums are added in LDS in a fixed order (no
//     atomics, so results are reproducible), then the fused epilogue and
//     8-byte stores;
//   * split-K (splits > 1, a grid of slabs x splits): when there are too few
//     slabs to fill the chip, each slab's K range is also divided over
//     `splits` workgroups, which pass their partial slabs through a
//     workspace; the last to arrive adds them in split order and finishes;
//   * stream-K (a grid of one workgroup per CU): the 32-k steps of all slabs
//     cut into equal contiguous ranges, shared slabs meeting in the same
//     workspace (gemm_skinny_streamk_kernel below).
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

// LDS of the kernel, per wave: RS floats, 32 KB with the preload (its slice
// of A, 16 rows x 32 PRE k), else 16 KB; after its k-loop, its RB 16 x 64
// fp32 partial sums (4 KB each) at red(wave, b, i, lane).  Each wave touches
// only its own region until the barrier before the cross-wave reduction.
template <bool BIG>
constexpr int region_floats() { return BIG ? 256 * PRE : 4096; }

template <bool BIG>
__device__ __forceinline__ float &red_at(u32x4 *smem, int w, int b, int i, int l) {
    return reinterpret_cast<float *>(smem)[region_floats<BIG>() * w + 1024 * b + 64 * i + l];
}

// Where a wave's k-loop takes A from (RB = 1 for the last two):
//   A_GLOBAL   16-byte loads from L2 in every step, beside B's;
//   A_PRELOAD  the wave's whole slice (PRE / 2 < steps <= PRE) into LDS by
//              direct loads, then into registers, before the loop;
//   A_STAGED   the wave's steps in chunks of at most PRE / RB (a multiple of
//              4): each chunk's slice of every row block into LDS by direct
//              loads, then one 16-byte LDS read per step and row block.
constexpr int A_GLOBAL = 0, A_PRELOAD = 1, A_STAGED = 2;

// RB: 16-row blocks of A (and C) per workgroup, 1..4 (M <= 16 RB).  Every
// block multiplies the same B vectors, so B is still read once; the preload
// path and split-K are for RB = 1 only.  One wave per SIMD gives a lane up
// to 512 registers: four blocks need more than the 256 of two waves per
// SIMD (with 8 waves they spilled and ran 2-3x slower than three blocks),
// and every instance ran as fast or faster on 4 waves than on 8 (M = 16,
// K = 4096 with the preload: 18.95 against 19.86 us).
//
// slab_part: the workgroup's sums over the 32-k steps [sp_begin, sp_begin +
// sp_len) of slab `slab`, left in every wave's LDS region; returns after the
// barrier that makes them visible to every wave.
template <class T, int AMODE, int RB>
__device__ __forceinline__ void slab_part(const GemmArgs &args, u32x4 *smem, int slab, int sp_begin, int sp_len) {
    static_assert(RB >= 1 && RB <= 4 && (RB == 1 || AMODE != A_PRELOAD), "row blocks");
    constexpr bool PRELOAD = AMODE == A_PRELOAD;
    constexpr bool BIG = AMODE != A_GLOBAL;
    constexpr int RS = region_floats<BIG>();
    const int M = args.M, N = args.N, K = args.K;
    const uint16_t *__restrict__ A = args.A;
    const uint16_t *__restrict__ B = args.B;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: loop control stays scalar
    const int p = lane & 15;
    const int h = lane >> 4;
    const int nb = slab * SLAB;
    const int ncol = nb + 4 * p;              // N % 4 == 0: all four columns valid or none

    // this workgroup's part of the slab's 32-k steps, divided over its waves
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
    } else if constexpr (AMODE == A_STAGED) {
        // Chunks of at most CH steps of the wave's range.  A chunk's slice of
        // each row block b goes to block b's part of the wave's LDS region
        // (CH / 4 pieces of 4 KB) by the direct loads of the preload (same
        // layout and swizzle), only its ceil(n / 4) groups of 4 steps: 4 rows
        // x 256 contiguous bytes per load, whole cache lines, where a
        // 16-byte A load per step takes half lines.  Steps past the chunk
        // read zero in both operands, and every group of 4 steps the loop
        // touches was loaded (so no stale LDS data reaches an MFMA).  The
        // chunk's first two batches of B go out around the A loads, as in
        // the preload.
        constexpr int CH = PRE / RB / 4 * 4;
        static_assert(CH >= 4 && RB * CH * 1024 <= 4 * RS, "staged slices fit the wave's region");
        const uint32_t region = lds_address(smem) + 4u * RS * (uint32_t)wave;
        const i32x4 rs = rsrc_words((const char *)A - ASHIFT, 2u * (uint32_t)M * (uint32_t)K + ASHIFT);
        const int r0 = lane >> 4;
        const int slot = lane & 15;
        for (int c0 = s_begin; c0 < s_end; c0 += CH) {
            const int cn = min(CH, s_end - c0);
            const int c_end = c0 + cn;
            auto load_b = [&](u32x2 (&vb)[UNROLL][8], int s0) __attribute__((always_inline)) {
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    const int kb = (s0 + u) * 32 + 8 * h;
                    const uint32_t mk = mask_of(s0 + u < c_end && kb < K);
                    const uint32_t boff = (uint32_t)kb * b_row + b_col;
#pragma unroll
                    for (int r = 0; r < 8; ++r)
                        vb[u][r] = __builtin_amdgcn_raw_buffer_load_b64(rb, (int)((boff + (uint32_t)r * b_row) | mk),
                                                                        0, CPOL_NT);
                }
            };
            // the 16-byte A fragment of row block b, chunk step i
            auto a_at = [&](int b, int i) __attribute__((always_inline)) {
                const uint32_t c = (uint32_t)((4 * (i & 3) + h) ^ p);
                return *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)(
                    region + 1024u * CH * (uint32_t)b + 4096u * (uint32_t)(i >> 2) + 256u * (uint32_t)p + 16u * c);
            };
            auto a_pair = [&](int i) __attribute__((always_inline)) {
                ABatch<RB> va;
#pragma unroll
                for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                    for (int b = 0; b < RB; ++b)
                        va.v[u][b] = a_at(b, i + u);
                return va;
            };
            load_b(vb0, c0);
            {
                const int kend = min(K, 32 * c_end);
#pragma unroll
                for (int b = 0; b < RB; ++b)
#pragma unroll
                    for (int c4 = 0; c4 < CH / 4; ++c4) {
                        if (4 * c4 < cn) {
#pragma unroll
                            for (int rq = 0; rq < 4; ++rq) {
                                // row 16 b + r of A; rows >= M lie past the buffer and read zero
                                const int r = 16 * b + 4 * rq + r0;
                                const int k = 32 * c0 + 128 * c4 + 8 * (slot ^ (r & 15));
                                const uint32_t off =
                                    (ASHIFT - 1024u * (uint32_t)rq + 2u * ((uint32_t)r * (uint32_t)K + (uint32_t)k)) +
                                    (k < kend ? 0u : 0x80000000u);
                                dma16_rq(rq, rs, off, region + 1024u * CH * (uint32_t)b + 4096u * (uint32_t)c4);
                            }
                        }
                    }
            }
            load_b(vb1, c0 + UNROLL);
            // the chunk's A loads are older than the second batch's 8 UNROLL B loads
            wait_vmcnt<8 * UNROLL>();
            for (int i = 0; i < cn; i += 2 * UNROLL) {
                if (i > 0)
                    load_b(vb1, c0 + i + UNROLL);
                __builtin_amdgcn_sched_barrier(0);
                mma_batch(vb0, a_pair(i));
                __builtin_amdgcn_sched_barrier(0);
                if (i + 2 * UNROLL < cn)
                    load_b(vb0, c0 + i + 2 * UNROLL);
                __builtin_amdgcn_sched_barrier(0);
                mma_batch(vb1, a_pair(i + UNROLL));
                __builtin_amdgcn_sched_barrier(0);
            }
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
                red_at<BIG>(smem, wave, b, 4 * e + j, lane) = acc[b][j][e];
    __syncthreads();
}

// The sum over the waves of (row block b, column group e) for this lane,
// in wave order.
template <bool BIG>
__device__ __forceinline__ void wave_sum(u32x4 *smem, int b, int e, int lane, float (&y)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w)
            s += red_at<BIG>(smem, w, b, 4 * e + j, lane);
        y[j] = s;
    }
}

// The epilogue and the 8-byte store of C[16 b + p][n .. n + 3], n = 64 slab
// + 16 h + 4 e, from the lane's four sums.
template <class T, int EPI>
__device__ __forceinline__ void finish(const GemmArgs &args, int slab, int b, int e, int lane, const float (&y)[4]) {
    const int p = lane & 15;
    const int h = lane >> 4;
    const int m = 16 * b + p;
    const int n = slab * SLAB + 16 * h + 4 * e;
    if (m >= args.M || n >= args.N)
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
    *reinterpret_cast<u32x2 *>(args.C + (uint32_t)m * (uint32_t)args.N + n) = u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
}

// One workgroup per slab (grid.x), its K range split over grid.y =
// ws.splits workgroups (split-K, RB = 1; 1: no split).
template <class T, int EPI, int AMODE, int RB>
__global__ __launch_bounds__(NTHREADS) void gemm_skinny_kernel(GemmArgs args, SplitWs ws) {
    constexpr bool BIG = AMODE != A_GLOBAL;
    __shared__ __attribute__((aligned(16))) u32x4 smem[WAVES * region_floats<BIG>() / 4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int steps = (args.K + 31) / 32;
    const int splits = ws.splits;
    const int split = blockIdx.y;
    const int sp_begin = (int)(((int64_t)steps * split) / splits);
    const int sp_len = (int)(((int64_t)steps * (split + 1)) / splits) - sp_begin;
    slab_part<T, AMODE, RB>(args, smem, blockIdx.x, sp_begin, sp_len);
    if constexpr (RB == 1) {
        // waves 0..3 each finish one of the four column groups e of every lane
        const int e = wave;
        float y[4];
        wave_sum<BIG>(smem, 0, e, lane, y);
        if (splits > 1 && !split_exchange(ws, blockIdx.x, split, y, e))
            return;
        finish<T, EPI>(args, blockIdx.x, 0, e, lane, y);
    } else {
        // the 4 RB (row block, column group) pairs are spread over the waves
#pragma unroll
        for (int q0 = 0; q0 < 4 * RB; q0 += WAVES) {
            const int q = q0 + wave;
            if (q < 4 * RB) {
                float y[4];
                wave_sum<BIG>(smem, q >> 2, q & 3, lane, y);
                finish<T, EPI>(args, blockIdx.x, q >> 2, q & 3, lane, y);
            }
        }
    }
}

// Stream-K (M <= 16): the slabs' 32-k steps, slab after slab, form one
// sequence of slabs x steps units, cut into gridDim.x equal contiguous
// ranges, one per workgroup.  A workgroup walks its range slab by slab: a
// slab it covers whole it finishes itself; its part of a slab it shares
// (at most two: the first and the last of its range) it publishes as a
// partial block, and after its whole range it counts its arrival at those
// slabs, the last to arrive adding the parts in K order and finishing.
// Deferring the arrivals to the end keeps the wait for the partial stores
// and the counter round trip out of the middle of the range.  Workgroup g's
// part of slab s has partial slot g + s (the (slab, workgroup) pairs in
// sequence order), so the slots of one slab are consecutive.  With every
// slab the same size, no CU holds more than ceil(slabs x steps /
// workgroups) steps, where an even split leaves CUs idle whenever the slab
// count does not divide the CU count (N = 11008: 172 slabs of 128 steps on
// 256 CUs, 86 steps per workgroup instead of 128).  Each wave stages its A
// slice through 32 KB of LDS, so one workgroup fills a CU: the limit per CU
// is its loads in flight, and two workgroups on one CU would leave another
// idle.
template <class T, int EPI>
__global__ __launch_bounds__(NTHREADS) void gemm_skinny_streamk_kernel(GemmArgs args, SplitWs ws) {
    __shared__ __attribute__((aligned(16))) u32x4 smem[WAVES * region_floats<true>() / 4];
    __shared__ uint32_t last_of[2];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t steps = (args.K + 31) / 32;
    const int64_t total = (int64_t)((args.N + SLAB - 1) / SLAB) * steps;
    const int64_t G = gridDim.x, g = blockIdx.x;
    // workgroup g covers units [g total / G, (g + 1) total / G); unit x lies
    // in the range of workgroup ((x + 1) G - 1) / total
    auto owner = [&](int64_t x) __attribute__((always_inline)) { return (int)(((x + 1) * G - 1) / total); };
    // the shared slabs of the range: slab, its first workgroup, its parts
    int sh_slab[2] = {0, 0}, sh_first[2] = {0, 0}, sh_parts[2] = {1, 1};
    int nsh = 0;
    const int64_t x1 = (g + 1) * total / G;
    for (int64_t x = g * total / G; x < x1;) {
        const int s = (int)(x / steps);
        const int64_t base = (int64_t)s * steps;
        const int64_t xe = x1 < base + steps ? x1 : base + steps;
        slab_part<T, A_STAGED, 1>(args, smem, s, (int)(x - base), (int)(xe - x));
        float y[4];
        wave_sum<true>(smem, 0, wave, lane, y);
        if (x == base && xe == base + steps) {
            finish<T, EPI>(args, s, 0, wave, lane, y);
        } else {
            const int first = owner(base);
            const int parts = owner(base + steps - 1) - first + 1;
            part_publish(ws.part + (int64_t)(first + s) * 1024, parts, (int)g - first, y, wave);
            if (nsh == 0) {
                sh_slab[0] = s, sh_first[0] = first, sh_parts[0] = parts;
            } else {
                sh_slab[1] = s, sh_first[1] = first, sh_parts[1] = parts;
            }
            ++nsh;
        }
        __syncthreads();   // every wave has read the LDS sums before the next part rewrites them
        x = xe;
    }
    if (nsh == 0)
        return;
    // the partial stores are complete before any arrival is counted
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        last_of[0] = part_arrive(ws.count + sh_slab[0], sh_parts[0]);
        if (nsh > 1)
            last_of[1] = part_arrive(ws.count + sh_slab[1], sh_parts[1]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if (i < nsh && last_of[i]) {
            float y[4];
            part_sum(ws.part + (int64_t)(sh_first[i] + sh_slab[i]) * 1024, sh_parts[i], y, wave);
            finish<T, EPI>(args, sh_slab[i], 0, wave, lane, y);
        }
    }
}

// The instances without the preload (row blocks, and one block where the
// preload does not apply) stage A through LDS in chunks, except where every
// wave has at most kGlobalASteps 32-k steps: there the chunk's start-up
// costs more than the half-line A loads.  Measured on an MI355X (fp16,
// rotating weight sets): 32 x 11008 x 4096 25.8 -> 22.2 us, 48 rows 30.0 ->
// 24.7 us, 64 rows 33.9 -> 26.7 us, 16 x 11008 x 8192 40.7 -> 37.9 us,
// 16 x 11008 x 11008 55.0 -> 50.8 us; 16 x 4096 x 4096 in 4 splits (8 steps
// per wave) 10.1 -> 10.5 us, hence the threshold.
constexpr int kGlobalASteps = 8;

template <class T, int EPI, int RB>
hipError_t launch_rows(const GemmArgs &a, const SplitWs &ws, hipStream_t stream) {
    const int slabs = (a.N + SLAB - 1) / SLAB;
    const int64_t steps = (a.K + 31) / 32;
    const int64_t hi = (steps + ws.splits - 1) / ws.splits;   // a split's share, rounded up
    if ((hi + WAVES - 1) / WAVES <= kGlobalASteps)
        hipLaunchKernelGGL((gemm_skinny_kernel<T, EPI, A_GLOBAL, RB>), dim3(slabs, ws.splits), dim3(NTHREADS), 0,
                           stream, a, ws);
    else
        hipLaunchKernelGGL((gemm_skinny_kernel<T, EPI, A_STAGED, RB>), dim3(slabs, ws.splits), dim3(NTHREADS), 0,
                           stream, a, ws);
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
    const int64_t steps = (a.K + 31) / 32;
    if (ws.streamk > 0) {   // 1 <= workgroups <= slabs x steps, checked by the host
        if ((int64_t)ws.streamk > slabs * steps)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL((gemm_skinny_streamk_kernel<T, EPI>), dim3(ws.streamk), dim3(NTHREADS), 0, stream, a, ws);
        return hipGetLastError();
    }
    // every wave's share of the 32-k steps is floor or ceil of a split's
    // share / WAVES, and a split's share floor or ceil of steps / splits
    const int64_t lo = steps / ws.splits, hi = (steps + ws.splits - 1) / ws.splits;
    if (lo / WAVES > PRE / 2 && (hi + WAVES - 1) / WAVES <= PRE)
        hipLaunchKernelGGL((gemm_skinny_kernel<T, EPI, A_PRELOAD, 1>), dim3(slabs, ws.splits), dim3(NTHREADS), 0, stream, a,
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
