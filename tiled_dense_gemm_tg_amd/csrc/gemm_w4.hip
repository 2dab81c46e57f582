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
// block (the wave reads 1 KiB contiguously) and 8 k of one A row, and runs
// four v_mfma_f32_16x16x32 with W^T as the 16-row operand (row l % 16 of MFMA
// j is column 16 j + l % 16) and A as the 16-column operand.  The MFMA
// multiplies the integers q - 8 (exact in both 16-bit formats), and the
// group's scale is applied once per group to the fp32 partial product, so
// each weight is rounded nowhere.  One group's loads are in flight while the
// previous group is multiplied; the waves' sums are added in LDS in a fixed
// order, then the fused epilogue and the stores.
#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int WAVES = 8;
constexpr int NTHREADS = 64 * WAVES;
constexpr uint32_t OOB = 0xFFFFFFF0u;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// `off` if ok, else an offset beyond every buffer.  The mask goes through an
// empty asm so the compiler keeps an OR instead of branching around the load
// (which would also make it wait for every load in flight).
__device__ __forceinline__ uint32_t masked(uint32_t off, bool ok) {
    uint32_t m = ok ? 0u : OOB;
    asm volatile("" : "+v"(m));
    return off | m;
}

// Pair m (m = 0..3) of the 8 nibbles: k-indices 2m (low half) and 2m+1 as
// 16-bit q - 8 values of the format of T.
template <class T>
__device__ __forceinline__ uint32_t dequant_pair(uint32_t x, int m) {
    const uint32_t magic = ((x >> (4 * m)) & 0x000F000Fu) | 0x64006400u;   // fp16 1024 + q
    const h2 v = __builtin_bit_cast(h2, magic) - h2{(_Float16)1032.0f, (_Float16)1032.0f};
    if constexpr (__is_same(T, F16)) {
        return __builtin_bit_cast(uint32_t, v);
    } else {
        // small integers: exact in bf16, whose bits are the top half of fp32
        const uint32_t lo = __builtin_bit_cast(uint32_t, (float)v.x);
        const uint32_t hi = __builtin_bit_cast(uint32_t, (float)v.y);
        return perm_hi(lo, hi);
    }
}

template <class T>
__device__ __forceinline__ u32x4 dequant8(uint32_t x) {
    return u32x4{dequant_pair<T>(x, 0), dequant_pair<T>(x, 1), dequant_pair<T>(x, 2), dequant_pair<T>(x, 3)};
}

// One scale group's operands for one lane: STEPS 32-k steps of packed W and A.
template <int STEPS>
struct GroupLoad {
    u32x4 w[STEPS];
    u32x4 a[STEPS];
    uint16_t s[4][4];   // [j][e] scale of column 16 j + 4 (l/16) + e
};

// SVEC: N % 4 == 0 and scales 8-byte aligned, so a lane's 4 consecutive
// columns of a scale row come in one 8-byte load.
template <class T, int EPI, int GROUP, bool SVEC>
__global__ __launch_bounds__(NTHREADS) void gemm_w4_kernel(GemmArgs args, const uint8_t *__restrict__ packed,
                                                          const uint16_t *__restrict__ scales) {
    constexpr int STEPS = GROUP / 32;
    __shared__ float red[WAVES][16][64];
    const int M = args.M, N = args.N, K = args.K;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = lane & 15;
    const int h = lane >> 4;
    const int slab = blockIdx.x;
    const int m0 = blockIdx.y * 16;
    const int ktiles = K / 32;
    const int groups = K / GROUP;
    const int g_begin = (int)(((int64_t)groups * wave) / WAVES);
    const int g_end = (int)(((int64_t)groups * (wave + 1)) / WAVES);

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

    auto load_group = [&](GroupLoad<STEPS> &g, int grp) __attribute__((always_inline)) {
        const bool live = grp < g_end;    // wave-uniform; past the range everything reads zero
#pragma unroll
        for (int u = 0; u < STEPS; ++u) {
            const uint32_t t = (uint32_t)(grp * STEPS + u);
            g.w[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)masked(w_base + 1024u * t, live), 0, 0);
            g.a[u] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)masked(a_row + 64u * t, a_ok && live), 0, 0);
        }
        if constexpr (SVEC) {
            // columns n .. n + 3 are all below N or all past it (N % 4 == 0)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n_lane + 16 * j;
                const uint32_t so = 2u * ((uint32_t)grp * (uint32_t)N + (uint32_t)n);
                const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)masked(so, live && n < N), 0, 0);
                g.s[j][0] = (uint16_t)(v.x & 0xffff);
                g.s[j][1] = (uint16_t)(v.x >> 16);
                g.s[j][2] = (uint16_t)(v.y & 0xffff);
                g.s[j][3] = (uint16_t)(v.y >> 16);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = n_lane + 16 * j + e;
                    const uint32_t so = 2u * ((uint32_t)grp * (uint32_t)N + (uint32_t)n);
                    g.s[j][e] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)masked(so, live && n < N), 0, 0);
                }
        }
    };

    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mma_group = [&](const GroupLoad<STEPS> &g) __attribute__((always_inline)) {
        f32x4 part[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            part[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < STEPS; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                part[j] = T::mfma16(dequant8<T>(g.w[u][j]), g.a[u], part[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[j][e] += T::to_f32(g.s[j][e]) * part[j][e];
    };

    GroupLoad<STEPS> b0, b1;
    load_group(b0, g_begin);
    for (int g = g_begin; g < g_end; g += 2) {
        load_group(b1, g + 1);
        __builtin_amdgcn_sched_barrier(0);
        mma_group(b0);
        __builtin_amdgcn_sched_barrier(0);
        if (g + 1 >= g_end)
            break;
        load_group(b0, g + 2);
        __builtin_amdgcn_sched_barrier(0);
        mma_group(b1);
        __builtin_amdgcn_sched_barrier(0);
    }

    // acc[j][e] = C[m0 + p][n_lane + 16 j + e] (this wave's groups)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            red[wave][4 * j + e][lane] = acc[j][e];
    __syncthreads();
    // waves 0..3 each finish one column group j of every lane
    if (wave >= 4)
        return;
    const int m = m0 + p;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        args.C, (short)0, (int)(2u * (uint32_t)M * (uint32_t)N), 0x00020000);
    {
        const int j = wave;
        const int n = n_lane + 16 * j;
        uint16_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float y = 0.f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w)
                y += red[w][4 * j + e][lane];
            float b = 0.f;
            if constexpr (EPI != EPI_NONE)
                b = n + e < N ? T::to_f32(args.bias[n + e]) : 0.f;
            o[e] = T::from_f32(epilogue<EPI>(y, b));
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

template <class T, int EPI, bool SVEC>
hipError_t launch_scales(const GemmArgs &a, const uint8_t *packed, const uint16_t *scales, int group,
                         hipStream_t stream) {
    const dim3 grid((a.N + 63) / 64, (a.M + 15) / 16);
    switch (group) {
    case 32:
        hipLaunchKernelGGL((gemm_w4_kernel<T, EPI, 32, SVEC>), grid, dim3(NTHREADS), 0, stream, a, packed, scales);
        break;
    case 64:
        hipLaunchKernelGGL((gemm_w4_kernel<T, EPI, 64, SVEC>), grid, dim3(NTHREADS), 0, stream, a, packed, scales);
        break;
    case 128:
        hipLaunchKernelGGL((gemm_w4_kernel<T, EPI, 128, SVEC>), grid, dim3(NTHREADS), 0, stream, a, packed, scales);
        break;
    default:
        hipLaunchKernelGGL((gemm_w4_kernel<T, EPI, 256, SVEC>), grid, dim3(NTHREADS), 0, stream, a, packed, scales);
        break;
    }
    return hipGetLastError();
}

template <class T, int EPI>
hipError_t launch_group(const GemmArgs &a, const uint8_t *packed, const uint16_t *scales, int group,
                        hipStream_t stream) {
    const bool svec = a.N % 4 == 0 && ((uintptr_t)scales & 7u) == 0;
    return svec ? launch_scales<T, EPI, true>(a, packed, scales, group, stream)
                : launch_scales<T, EPI, false>(a, packed, scales, group, stream);
}

template <class T>
hipError_t launch_epi(int epi, const GemmArgs &a, const uint8_t *packed, const uint16_t *scales, int group,
                      hipStream_t stream) {
    switch (epi) {
    case EPI_NONE: return launch_group<T, EPI_NONE>(a, packed, scales, group, stream);
    case EPI_BIAS: return launch_group<T, EPI_BIAS>(a, packed, scales, group, stream);
    default: return launch_group<T, EPI_BIAS_GELU_TANH>(a, packed, scales, group, stream);
    }
}

}  // namespace

hipError_t launch_w4(int dtype, int epi, const GemmArgs &a, const uint8_t *packed, const uint16_t *scales, int group,
                     hipStream_t stream) {
    return dtype == 0 ? launch_epi<F16>(epi, a, packed, scales, group, stream)
                      : launch_epi<BF16>(epi, a, packed, scales, group, stream);
}

hipError_t launch_w4_pack(int K, int N, const uint8_t *q, uint8_t *packed, hipStream_t stream) {
    const int64_t dwords = (int64_t)((N + 63) / 64) * K * 8;   // 1 KiB = 256 dwords per 32 k x 64 n
    const int64_t blocks = (dwords + 255) / 256;
    hipLaunchKernelGGL(w4_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, K, N, q,
                       reinterpret_cast<uint32_t *>(packed), dwords);
    return hipGetLastError();
}

}  // namespace tg
