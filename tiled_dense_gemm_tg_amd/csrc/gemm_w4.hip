// gemm_w4.hip -- weight-only 4-bit GEMM for gfx950: C = epi(A * W [+ bias])
// with W[k][n] = (q[k][n] - 8) * s[k / group][n], q in 0..15.
//
// The first TileLang page ("TileLang: writing LLM GPU kernels by thinking in
// tiles", section 5, "Quantized LLM inference") describes this pattern: the
// weights stay compressed in memory, are turned back into 16-bit values in
// registers and go straight into the matrix product, instead of a separate
// dequantization pass that writes 16-bit weights out and reads them back.
// With few rows of A (decode-shaped products) the work is bound by reading
// W, so 4-bit weights move a quarter of the bytes of 16-bit ones.
//
// Packed layout (written by w4_pack_kernel, read here): 1 KiB blocks of
// 32 k x 64 n, block (slab s, k-tile t) at byte 1024 (s * K/32 + t), so the
// k-tiles of one 64-column slab are contiguous.  In a block, lane l owns
// 16 bytes at 16 l; its dword j holds column n = 64 s + 16 j + l % 16 at the
// 8 k = 32 t + 8 (l / 16) + i, with k-index i in nibble p(i) = i / 2 + 4 (i % 2).
// That order lets one shift and one and-or per pair of k produce the two
// 16-bit values of an MFMA operand dword (1024 + q as fp16 bits), and one
// packed fp16 subtract of 1032 gives q - 8 exactly.
//
// Work: one workgroup per (16-row block of A, 64-column slab); its 8 waves
// split the scale groups.  Per 32-k step a lane loads its 16 bytes of the
// block (the wave reads 1 KiB contiguously) and 8 k of one A row (from the
// wave's copy of its A slice in LDS where every wave has 9 to 16 steps and
// the groups are at least 64 k; see LDSA below), and runs
// four v_mfma_f32_16x16x32 with W^T as the 16-row operand (row l % 16 of MFMA
// j is column 16 j + l % 16) and A as the 16-column operand.  The MFMA
// multiplies the integers q - 8 (exact in both 16-bit formats), and the
// group's scale is applied once per group to the fp32 partial product, so
// each weight is rounded nowhere.  Each wave keeps 16 steps' loads in flight
// (8 with 32-k groups) in a ring of scale groups, refilling a group's slot as
// soon as it has been multiplied; the waves' sums are added in LDS in a fixed
// order, then the fused epilogue and the stores.  With split-K (splits > 1,
// a grid of slabs x row blocks x splits) each workgroup takes a part of the
// scale groups and the partial blocks meet through the workspace.
#include "tg_device.h"
#include "tg_launch.h"
#include "tg_direct.h"
#include "tg_split.h"

namespace tg {
namespace {

using namespace direct;

constexpr int WAVES = 8;
constexpr int NTHREADS = 64 * WAVES;
constexpr uint32_t OOB = 0xFFFFFFF0u;
constexpr uint32_t ASHIFT = 4096;        // the staged-A buffer starts this far before A
// Cache policy of the weight and scale loads: non-temporal (each is read
// once; A is what the workgroups re-read from L2).
constexpr int CPOL_NT = 2;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// `off` if ok, else an offset beyond every buffer.  The mask goes through an
// empty asm so the compiler keeps an OR instead of branching around the load
// (which would also make it wait for every load in flight).
__device__ __forceinline__ uint32_t masked(uint32_t off, bool ok) {
    uint32_t m = ok ? 0u : OOB;
    asm volatile("" : "+v"(m));
    return off | m;
}

// (x & mask) | bits in one instruction (the two constants stay in registers:
// a three-operand instruction takes no literal here).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(bits));
    return r;
}

// The 8 nibbles of x as 16-bit q - 8 values of the format of T, pair m
// (k-indices 2m in the low half, 2m+1 in the high half) from the nibbles at
// bits 4m and 16 + 4m.
template <class T>
__device__ __forceinline__ u32x4 dequant8(uint32_t x, uint32_t magic) {
    if constexpr (__is_same(T, F16)) {
        // A nibble at bits 0..3 of a half under the fp16 pattern of 1024 reads
        // 1024 + q, at bits 4..7 it reads 1024 + 16 q; one packed subtract, or
        // one packed multiply-add by 1/16 and -72, gives q - 8 (all exact).
        // Pairs 2 and 3 use the same two masks on x >> 8.
        const uint32_t y = x >> 8;
        const h2 sub = {(_Float16)-1032.0f, (_Float16)-1032.0f};
        const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
        const h2 off = {(_Float16)-72.0f, (_Float16)-72.0f};
        const h2 p0 = __builtin_bit_cast(h2, and_or(x, 0x000F000Fu, magic)) + sub;
        const h2 p1 = __builtin_bit_cast(h2, and_or(x, 0x00F000F0u, magic)) * sixteenth + off;
        const h2 p2 = __builtin_bit_cast(h2, and_or(y, 0x000F000Fu, magic)) + sub;
        const h2 p3 = __builtin_bit_cast(h2, and_or(y, 0x00F000F0u, magic)) * sixteenth + off;
        return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                     __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
    } else {
        // through fp16 as above, then widened: small integers are exact in
        // bf16, whose bits are the top half of fp32
        u32x4 r;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const h2 v = __builtin_bit_cast(h2, and_or(x >> (4 * m), 0x000F000Fu, magic)) -
                         h2{(_Float16)1032.0f, (_Float16)1032.0f};
            r[m] = perm_hi(__builtin_bit_cast(uint32_t, (float)v.x), __builtin_bit_cast(uint32_t, (float)v.y));
        }
        return r;
    }
}

// One scale group's operands for one lane: STEPS 32-k steps of packed W and
// A, and the scales of its 16 columns, [j][e] for column 16 j + 4 (l/16) + e
// (SVEC: two per dword, e = 2 i + half).
template <int STEPS, bool SVEC>
struct GroupLoad {
    u32x4 w[STEPS];
    u32x4 a[STEPS];
    u32x2 sv[SVEC ? 4 : 1];
    uint16_t s[SVEC ? 1 : 4][4];
};

// SVEC: N % 4 == 0 and scales 8-byte aligned, so a lane's 4 consecutive
// columns of a scale row come in one 8-byte load.
// LDSA: every wave's share of A is at most 16 steps (the host picks this
// instance only then, and only with SVEC and groups of at least 64 k) and is
// staged once through the wave's LDS region by direct loads, each of 4 rows
// x 256 contiguous bytes (half the cache lines of the 16 rows x 64 bytes a
// step's A fragment spans), instead of riding in the ring of loads.
template <class T, int EPI, int GROUP, bool SVEC, bool LDSA>
__global__ __launch_bounds__(NTHREADS) void gemm_w4_kernel(GemmArgs args, const uint8_t *__restrict__ packed,
                                                          const uint16_t *__restrict__ scales, SplitWs ws) {
    constexpr int STEPS = GROUP / 32;
    // groups in flight per wave: 16 steps' loads, or 8 where the scales take
    // as many registers as the weights (32-k groups, element-wise scale
    // loads), and at least two groups
    constexpr int RING_STEPS = (SVEC && GROUP >= 64) ? 16 : 8;
    constexpr int RING = RING_STEPS / STEPS >= 2 ? RING_STEPS / STEPS : 2;
    static_assert(!LDSA || (SVEC && GROUP >= 64), "staged A goes with 16-step rings");
    // per wave: its staged slice of A (LDSA), then its 16 x 64 fp32 partial
    // sums (the first 4 KB), each wave touching only its own region until
    // the barrier before the cross-wave reduction
    constexpr int REGION = LDSA ? 16384 : 4096;
    __shared__ __attribute__((aligned(16))) u32x4 smem[WAVES * REGION / 16];
    auto red = [&](int w, int i, int l) __attribute__((always_inline)) -> float & {
        return reinterpret_cast<float *>(smem)[REGION / 4 * w + 64 * i + l];
    };
    const int M = args.M, N = args.N, K = args.K;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = lane & 15;
    const int h = lane >> 4;
    const int slab = blockIdx.x;
    const int m0 = blockIdx.y * 16;
    const int ktiles = K / 32;
    // this workgroup's scale groups (all of them without split-K), divided
    // over its waves
    const int groups = K / GROUP;
    const int splits = ws.splits;
    const int split = blockIdx.z;
    const int sp_begin = (int)(((int64_t)groups * split) / splits);
    const int sp_len = (int)(((int64_t)groups * (split + 1)) / splits) - sp_begin;
    const int g_begin = sp_begin + (int)(((int64_t)sp_len * wave) / WAVES);
    const int g_end = sp_begin + (int)(((int64_t)sp_len * (wave + 1)) / WAVES);

    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(args.A), (short)0,
                                          (int)(2u * (uint32_t)M * (uint32_t)K), 0x00020000);
    const uint32_t n_slabs = (uint32_t)((N + 63) / 64);
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(packed), (short)0,
                                          (int)(n_slabs * (uint32_t)K * 32u), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(scales), (short)0,
                                          (int)(2u * (uint32_t)groups * (uint32_t)N), 0x00020000);
    // rows of A past M read zero (pushed out of range)
    const bool a_ok = m0 + p < M;
    const uint32_t a_row = 2u * (uint32_t)(m0 + p) * (uint32_t)K + 16u * (uint32_t)h;
    const uint32_t w_base = 1024u * (uint32_t)slab * (uint32_t)ktiles + 16u * (uint32_t)lane;
    const int n_lane = slab * 64 + 4 * h;   // + 16 j + e

    auto load_group = [&](GroupLoad<STEPS, SVEC> &g, int grp) __attribute__((always_inline)) {
        const bool live = grp < g_end;    // wave-uniform; past the range everything reads zero
#pragma unroll
        for (int u = 0; u < STEPS; ++u) {
            const uint32_t t = (uint32_t)(grp * STEPS + u);
            g.w[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)masked(w_base + 1024u * t, live), 0, CPOL_NT);
            if constexpr (!LDSA)
                g.a[u] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)masked(a_row + 64u * t, a_ok && live), 0,
                                                               0);
        }
        if constexpr (SVEC) {
            // columns n .. n + 3 are all below N or all past it (N % 4 == 0)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n_lane + 16 * j;
                const uint32_t so = 2u * ((uint32_t)grp * (uint32_t)N + (uint32_t)n);
                g.sv[j] = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)masked(so, live && n < N), 0, CPOL_NT);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = n_lane + 16 * j + e;
                    const uint32_t so = 2u * ((uint32_t)grp * (uint32_t)N + (uint32_t)n);
                    g.s[j][e] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)masked(so, live && n < N), 0, CPOL_NT);
                }
        }
    };

    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t magic = 0x64006400u;   // fp16 1024 in both halves
    // staged A: step i of the wave's slice, row p, logical 16-byte chunk
    // 4 (i % 4) + h of 128-k block i / 4, at slot chunk ^ p of the row
    const uint32_t region = lds_address(smem) + (uint32_t)REGION * (uint32_t)wave;
    const uint32_t a_lds = region + 256u * (uint32_t)p;
    const uint32_t hp = (uint32_t)(h ^ p);
    auto mma_group = [&](const GroupLoad<STEPS, SVEC> &g, int grp) __attribute__((always_inline)) {
        f32x4 part[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            part[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x4 av[STEPS];
#pragma unroll
        for (int u = 0; u < STEPS; ++u) {
            if constexpr (LDSA) {
                const uint32_t i = (uint32_t)((grp - g_begin) * STEPS + u);
                av[u] = *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)(
                    a_lds + 4096u * (i >> 2) + 16u * (hp ^ (4u * (i & 3u))));
            } else {
                av[u] = g.a[u];
            }
        }
#pragma unroll
        for (int u = 0; u < STEPS; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                part[j] = T::mfma16(dequant8<T>(g.w[u][j], magic), av[u], part[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint16_t sb;
                if constexpr (SVEC)
                    sb = (uint16_t)(g.sv[j][e >> 1] >> (16 * (e & 1)));
                else
                    sb = g.s[j][e];
                acc[j][e] += T::to_f32(sb) * part[j][e];
            }
    };

    // A ring of RING groups: each group's slot is refilled with the group
    // RING places further on as soon as it has been multiplied.
    if constexpr (LDSA) {
        // Load j = 4 c4 + rq: row r = 4 rq + lane / 16 of the block, k = the
        // slice's first k + 128 c4 + 8 c, where the lane's slot lane % 16 of
        // the row holds logical chunk c = slot ^ r; LDS byte 4096 c4 + 256 r
        // + 16 slot of the region.  Chunks past the wave's range or K and
        // rows >= M are out of range and read zero.
        const i32x4 rsa = rsrc_words((const char *)args.A - ASHIFT, 2u * (uint32_t)M * (uint32_t)K + ASHIFT);
        const int r0 = lane >> 4;
        const int slot = lane & 15;
        const int k_first = 32 * STEPS * g_begin;
        const int kend = min(K, 32 * STEPS * g_end);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int r = 4 * rq + r0;
                const int k = k_first + 128 * c4 + 8 * (slot ^ r);
                const uint32_t off =
                    (ASHIFT - 1024u * (uint32_t)rq + 2u * ((uint32_t)(m0 + r) * (uint32_t)K + (uint32_t)k)) +
                    (k < kend ? 0u : 0x80000000u);
                dma16_rq(rq, rsa, off, region + 4096u * (uint32_t)c4);
            }
        }
    }
    GroupLoad<STEPS, SVEC> ring[RING];
#pragma unroll
    for (int r = 0; r < RING; ++r)
        load_group(ring[r], g_begin + r);
    if constexpr (LDSA) {
        // the 16 A loads are older than the ring's STEPS + 4 loads per group
        wait_vmcnt<RING * (STEPS + 4)>();
    }
    int g = g_begin;
    for (; g + RING < g_end; g += RING) {
#pragma unroll
        for (int r = 0; r < RING; ++r) {
            __builtin_amdgcn_sched_barrier(0);
            mma_group(ring[r], g + r);
            __builtin_amdgcn_sched_barrier(0);
            load_group(ring[r], g + RING + r);
        }
    }
#pragma unroll
    for (int r = 0; r < RING; ++r) {
        __builtin_amdgcn_sched_barrier(0);
        if (g + r < g_end)
            mma_group(ring[r], g + r);
    }

    // acc[j][e] = C[m0 + p][n_lane + 16 j + e] (this wave's groups)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            red(wave, 4 * j + e, lane) = acc[j][e];
    __syncthreads();
    // waves 0..3 each finish one column group j of every lane
    const int j = wave & 3;
    float y[4] = {0.f, 0.f, 0.f, 0.f};
    if (wave < 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int w = 0; w < WAVES; ++w)
                y[e] += red(w, 4 * j + e, lane);
    }
    if (splits > 1 && !split_exchange(ws, (int64_t)blockIdx.y * gridDim.x + blockIdx.x, split, y, j))
        return;
    if (wave >= 4)
        return;
    const int m = m0 + p;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        args.C, (short)0, (int)(2u * (uint32_t)M * (uint32_t)N), 0x00020000);
    {
        const int n = n_lane + 16 * j;
        uint16_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float b = 0.f;
            if constexpr (EPI != EPI_NONE)
                b = n + e < N ? T::to_f32(args.bias[n + e]) : 0.f;
            o[e] = T::from_f32(epilogue<EPI>(y[e], b));
        }
        const uint32_t base = 2u * ((uint32_t)m * (uint32_t)N + (uint32_t)n);
        if (n + 3 < N) {
            const uint32_t off = m < M ? base : OOB;
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])}, rc, (int)off, 0, 0);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t off = (m < M && n + e < N) ? base + 2u * e : OOB;
                __builtin_amdgcn_raw_buffer_store_b16(o[e], rc, (int)off, 0, 0);
            }
        }
    }
}

// One thread per packed dword: block (s, t), lane l, dword j.  Columns past
// N get q = 8 (weight 0).
__global__ __launch_bounds__(256) void w4_pack_kernel(int K, int N, const uint8_t *__restrict__ q,
                                                      uint32_t *__restrict__ out, int64_t dwords) {
    const int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (d >= dwords)
        return;
    const int j = (int)(d & 3);
    const int l = (int)((d >> 2) & 63);
    const int64_t block = d >> 8;
    const int ktiles = K / 32;
    const int t = (int)(block % ktiles);
    const int s = (int)(block / ktiles);
    const int n = 64 * s + 16 * j + (l & 15);
    const int k0 = 32 * t + 8 * (l >> 4);
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t v = n < N ? (uint32_t)(q[(int64_t)(k0 + i) * N + n] & 15u) : 8u;
        x |= v << (4 * ((i >> 1) + 4 * (i & 1)));
    }
    out[d] = x;
}

template <class T, int EPI, int GROUP, bool SVEC>
void launch_one(const GemmArgs &a, const uint8_t *packed, const uint16_t *scales, const SplitWs &ws,
                hipStream_t stream) {
    const dim3 grid((a.N + 63) / 64, (a.M + 15) / 16, ws.splits);
    // staged A when every wave's groups span at most 16 steps (and more than
    // 8, so the 128 KB of LDS pays): a wave gets floor or ceil of a split's
    // groups / WAVES, a split floor or ceil of groups / splits
    bool ldsa = false;
    if constexpr (SVEC && GROUP >= 64) {
        const int64_t groups = a.K / GROUP;
        const int64_t lo = groups / ws.splits, hi = (groups + ws.splits - 1) / ws.splits;
        ldsa = (lo / WAVES) * (GROUP / 32) > 8 && ((hi + WAVES - 1) / WAVES) * (GROUP / 32) <= 16;
    }
    if (ldsa)
        hipLaunchKernelGGL((gemm_w4_kernel<T, EPI, GROUP, SVEC, SVEC && GROUP >= 64>), grid, dim3(NTHREADS), 0,
                           stream, a, packed, scales, ws);
    else
        hipLaunchKernelGGL((gemm_w4_kernel<T, EPI, GROUP, SVEC, false>), grid, dim3(NTHREADS), 0, stream, a, packed,
                           scales, ws);
}

template <class T, int EPI, bool SVEC>
hipError_t launch_scales(const GemmArgs &a, const uint8_t *packed, const uint16_t *scales, int group,
                         const SplitWs &ws, hipStream_t stream) {
    switch (group) {
    case 32: launch_one<T, EPI, 32, SVEC>(a, packed, scales, ws, stream); break;
    case 64: launch_one<T, EPI, 64, SVEC>(a, packed, scales, ws, stream); break;
    case 128: launch_one<T, EPI, 128, SVEC>(a, packed, scales, ws, stream); break;
    default: launch_one<T, EPI, 256, SVEC>(a, packed, scales, ws, stream); break;
    }
    return hipGetLastError();
}

template <class T, int EPI>
hipError_t launch_group(const GemmArgs &a, const uint8_t *packed, const uint16_t *scales, int group,
                        const SplitWs &ws, hipStream_t stream) {
    const bool svec = a.N % 4 == 0 && ((uintptr_t)scales & 7u) == 0;
    return svec ? launch_scales<T, EPI, true>(a, packed, scales, group, ws, stream)
                : launch_scales<T, EPI, false>(a, packed, scales, group, ws, stream);
}

template <class T>
hipError_t launch_epi(int epi, const GemmArgs &a, const uint8_t *packed, const uint16_t *scales, int group,
                      const SplitWs &ws, hipStream_t stream) {
    switch (epi) {
    case EPI_NONE: return launch_group<T, EPI_NONE>(a, packed, scales, group, ws, stream);
    case EPI_BIAS: return launch_group<T, EPI_BIAS>(a, packed, scales, group, ws, stream);
    default: return launch_group<T, EPI_BIAS_GELU_TANH>(a, packed, scales, group, ws, stream);
    }
}

}  // namespace

hipError_t launch_w4(int dtype, int epi, const GemmArgs &a, const uint8_t *packed, const uint16_t *scales, int group,
                     const SplitWs &ws, hipStream_t stream) {
    return dtype == 0 ? launch_epi<F16>(epi, a, packed, scales, group, ws, stream)
                      : launch_epi<BF16>(epi, a, packed, scales, group, ws, stream);
}

hipError_t launch_w4_pack(int K, int N, const uint8_t *q, uint8_t *packed, hipStream_t stream) {
    const int64_t dwords = (int64_t)((N + 63) / 64) * K * 8;   // 1 KiB = 256 dwords per 32 k x 64 n
    const int64_t blocks = (dwords + 255) / 256;
    hipLaunchKernelGGL(w4_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, K, N, q,
                       reinterpret_cast<uint32_t *>(packed), dwords);
    return hipGetLastError();
}

}  // namespace tg
