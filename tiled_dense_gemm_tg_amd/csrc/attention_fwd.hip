// attention_fwd.hip -- FlashAttention forward for gfx950: O = softmax(scale Q K^T) V
// per (batch, head), BSHD layout, head dim 128, fp16 or bf16, fp32 accumulate.
//
// The TileLang pages present this as the kernel where tiles matter most
// ("TileLang: writing LLM GPU kernels by thinking in tiles", section 5,
// "FlashAttention"; "TileLang: you write the dataflow, the compiler owns the
// schedule", "FlashAttention, in tiles"): a block of queries stays on chip,
// key/value blocks stream past it, the scores of each block go through an
// online softmax (running row maximum, rescaling of the partial output,
// running sum of exponentials, exp2 with log2(e) folded into the scale) and
// straight into the second product, so the Sq x Sk score matrix never exists
// in memory.  The CDNA4 design:
//
//   * a workgroup of 8 waves holds 256 queries of one (batch, head); each
//     wave owns 32 of them, its Q fragments in registers for the whole loop
//     and its 32 x 128 output in 64 fp32 registers; two waves share each
//     SIMD, so one wave's softmax arithmetic overlaps the other's MFMAs;
//   * key/value blocks of 128 tokens stream through a 2-stage LDS ring
//     (128 KiB) by direct-to-LDS loads, each block requested one block
//     ahead, one barrier per block;
//   * both products are computed transposed on v_mfma_f32_32x32x16:
//     S^T = K Q^T (K rows from LDS, Q^T from registers) and
//     O^T = V^T P^T (V^T through the transposing LDS read), so every lane
//     holds the scores and the output of one query column: the row maximum
//     and sum need one exchange between the two lane halves, the rescaling
//     factor is per lane, and the probabilities go from the S accumulators
//     straight into the second MFMA's operand (the two halves of a lane's 8
//     keys are 4-key groups, and V^T is read in the same key order);
//   * rescaling is lazy: the running maximum used in the exponentials only
//     moves when a block's maximum exceeds it by more than 8 (in log2 units),
//     which keeps every exponential below 2^8 and rescales the output rarely;
//     numerator and denominator always share the same maximum, so the
//     quotient is unchanged;
//   * causal masking (query i sees keys 0..i, Sq == Sk) and the key tail
//     (k >= Sk) set scores to -inf in the blocks that need it; causal
//     workgroups stop at their last visible block, and the query blocks with
//     the most keys, over all heads, are dispatched first.
#include "tg_device.h"
#include "tg_direct.h"
#include "tg_launch.h"

#include <type_traits>
#include <utility>

namespace tg {
namespace {

constexpr int HD = 128;                   // head dim
constexpr int WAVES = 8;
constexpr int NTHREADS = 64 * WAVES;
constexpr int QW = 32;                    // queries per wave
constexpr int BM = QW * WAVES;            // queries per workgroup
constexpr int BN = 128;                   // keys per block
constexpr int STAGES = 2;
constexpr int KV_BYTES = BN * HD * 2;     // 32 KiB: one block of K (or V) in LDS
constexpr int STAGE_BYTES = 2 * KV_BYTES;
constexpr uint32_t SHIFT = 4096;          // buffers start 4 KiB before K and V
constexpr uint32_t OOB_BUMP = 0x80000000u;
constexpr float RESCALE_LOG2 = 8.0f;

using namespace direct;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// K rows are 256 bytes = 16 chunks; the fragment read takes one chunk of 32
// consecutive rows, so the chunk index is XOR-ed with row % 16.
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
// V rows are read transposed, 4 consecutive rows per pass (as B in the GEMM).
__device__ __forceinline__ int v_swz(int row) { return ((row & 1) ? 10 : 0) ^ ((row & 2) ? 4 : 0); }

typedef __attribute__((address_space(3))) const char *lds_ptr;

// Fragment reads at an LDS pointer plus a compile-time offset, which the
// assembler takes as the instruction's offset field.
__device__ __forceinline__ u32x4 lds_u4_at(lds_ptr p) {
    return *(__attribute__((address_space(3))) const u32x4 *)p;
}
__device__ __forceinline__ u32x2 lds_tr_at(lds_ptr p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
    return __builtin_bit_cast(u32x2, v);
}

// Two probabilities rounded to the 16-bit format (nearest even) and packed,
// and the sum of the two rounded values added to acc.
template <class T> struct Prob;
template <> struct Prob<F16> {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, h2));
    }
    static __device__ __forceinline__ float add_pair(uint32_t p, float acc) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, p), h2{(_Float16)1.0f, (_Float16)1.0f}, acc, false);
    }
};
template <> struct Prob<BF16> {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, b2));
    }
    static __device__ __forceinline__ float add_pair(uint32_t p, float acc) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, p), b2{(__bf16)1.0f, (__bf16)1.0f}, acc,
                                               false);
    }
};

__device__ __forceinline__ u32x4 lds_u4(uint32_t byte) {
    return *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)byte;
}

__device__ __forceinline__ u32x2 lds_tr(uint32_t byte) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)byte);
    return __builtin_bit_cast(u32x2, v);
}

// The maximum and the sum of x over lanes l and l ^ 32, in every lane, from
// v_permlane32_swap (a VALU exchange of one register's lanes 32-63 with
// another's lanes 0-31, no LDS round trip): with x in both registers, the
// first ends up holding the lower half's x in both halves and the second the
// upper half's, and one more VALU op combines them.  Written as assembly
// because the compiler's builtin for the instruction returns its first
// result for both at -O3; the combining op sits in the same block so the
// compiler adds no NaN-quieting ops around an opaque result.  Two wait
// states separate the exchange from the VALU write of its operands and from
// the VALU read of its results.
__device__ __forceinline__ float max_of_halves(float x) {
    float a = x, b = x;
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1" : "+v"(a), "+v"(b));
    return a;
}
__device__ __forceinline__ float sum_of_halves(float x) {   // lower half's x + upper half's x
    float a = x, b = x;
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_add_f32 %0, %0, %1" : "+v"(a), "+v"(b));
    return a;
}

template <class T, bool CAUSAL>
__global__ __launch_bounds__(NTHREADS, 1) void attention_fwd_kernel(AttnArgs args) {
    __shared__ __attribute__((aligned(16))) u32x4 smem[STAGES * STAGE_BYTES / 16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // One flat grid in which consecutive workgroups take the same query
    // block of consecutive (batch, head) pairs.  The XCDs take workgroups in
    // turn, so with B * H a multiple of the 8 XCDs every query block of a
    // head runs on one XCD and reads that head's K and V through one L2
    // (query blocks of one head spread over all XCDs fetched K and V once
    // per XCD).  Causal: the heaviest query blocks (longest key range) come
    // first, so the longest workgroups start earliest.
    const int bh = args.B * args.H;
    const int nqb = (int)gridDim.x / bh;
    const int id = (int)blockIdx.x;
    const int qb = CAUSAL ? nqb - 1 - id / bh : id / bh;
    const int h = (id % bh) % args.H;
    const int b = (id % bh) / args.H;
    const int q0 = qb * BM;
    const int Sq = args.Sq, Sk = args.Sk, H = args.H;
    const uint32_t tok = 2u * (uint32_t)H * (uint32_t)HD;   // bytes between tokens
    const uint32_t lds0 = lds_address(smem);
    auto stage = [&](int st) { return lds0 + (uint32_t)st * (uint32_t)STAGE_BYTES; };
    const int lh = lane >> 5;    // lane half
    const int lc = lane & 31;    // query column within a sub-tile

    // ---- Q fragments, d-step s: query qi = q0 + 32 wave + lc, d = 16 s + 8 lh .. +7
    const int qi = q0 + QW * wave + lc;
    u32x4 qf[8];
    {
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(args.Q), (short)0, (int)((uint32_t)args.B * (uint32_t)Sq * tok), 0x00020000);
        const uint32_t base = ((uint32_t)b * (uint32_t)Sq + (uint32_t)qi) * tok + 2u * (uint32_t)h * HD;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const uint32_t off = qi < Sq ? base + 2u * (uint32_t)(16 * s + 8 * lh) : 0xFFFFFFF0u;
            qf[s] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)off, 0, 0);
        }
    }

    // The Q loads are the only loads the compiler tracks here; waiting for them
    // now keeps it from waiting for every load in flight inside the loop.
    wait_vmcnt<0>();

    // ---- direct loads of one key/value block: wave w fills rows 16 w .. 16 w + 15
    // of K and of V, 4 instructions each (4 rows of 256 bytes per instruction).
    const uint32_t kv_bytes = (uint32_t)args.B * (uint32_t)Sk * tok;
    const i32x4 rk = rsrc_words((const char *)args.K - SHIFT, kv_bytes + SHIFT);
    const i32x4 rv = rsrc_words((const char *)args.V - SHIFT, kv_bytes + SHIFT);
    uint32_t koff[4], voff[4];
    int krow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * i + (lane >> 4);
        krow[i] = row;
        const uint32_t tok_base = ((uint32_t)b * (uint32_t)Sk + (uint32_t)row) * tok + 2u * (uint32_t)h * HD;
        koff[i] = SHIFT - 1024u * i + tok_base + 16u * (uint32_t)((lane & 15) ^ k_swz(row));
        voff[i] = SHIFT - 1024u * i + tok_base + 16u * (uint32_t)((lane & 15) ^ v_swz(row));
    }
    const uint32_t m0_k = 4096u * (uint32_t)wave;
    auto issue_block = [&](int blk, int st) __attribute__((always_inline)) {
        const int kb = blk * BN;
        const uint32_t adv = (uint32_t)kb * tok;
        const uint32_t sb = stage(st);
        auto one = [&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            const uint32_t mask = kb + krow[i] < Sk ? 0u : OOB_BUMP;
            dma16<1024 * i>(rk, koff[i] + adv + mask, sb + m0_k);
        };
        auto onev = [&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            const uint32_t mask = kb + krow[i] < Sk ? 0u : OOB_BUMP;
            dma16<1024 * i>(rv, voff[i] + adv + mask, sb + (uint32_t)KV_BYTES + m0_k);
        };
        one(std::integral_constant<int, 0>{});
        one(std::integral_constant<int, 1>{});
        one(std::integral_constant<int, 2>{});
        one(std::integral_constant<int, 3>{});
        onev(std::integral_constant<int, 0>{});
        onev(std::integral_constant<int, 1>{});
        onev(std::integral_constant<int, 2>{});
        onev(std::integral_constant<int, 3>{});
    };

    // ---- fragment read addresses (bytes within a stage)
    // K for S^T: key row 32 kt + lc, chunk 2 s + lh
    uint32_t ka[2][8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int row = 32 * kt + lc;
            ka[kt][s] = 256u * (uint32_t)row + 16u * (uint32_t)((2 * s + lh) ^ k_swz(row));
        }
    // V^T for O^T, d-tile dt, key step u: two transposed reads, key rows
    // 16 u + 4 lh + (0..3) and 16 u + 8 + 4 lh + (0..3), columns 32 dt + lc.
    const int G = lane >> 4;
    const int qq = lane & 15;
    uint32_t va[4];     // [dt], for u = 0, first read; + 256 * 16 u per step, + 2048 for the second read
    {
        const int row = 4 * (G >> 1) + (qq >> 2);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const int chunk = 4 * dt + 2 * (G & 1) + ((qq & 3) >> 1);
            va[dt] = (uint32_t)KV_BYTES + 256u * (uint32_t)row + 16u * (uint32_t)(chunk ^ v_swz(row)) +
                     8u * (uint32_t)(qq & 1);
        }
    }

    // per-lane read pointers into the current stage: K fragment s of the
    // first half, V^T tile dt of the first key step (the other halves and
    // steps are compile-time offsets); they move to the next stage after
    // every block
    lds_ptr kp[8], vp[4];
#pragma unroll
    for (int s = 0; s < 8; ++s)
        kp[s] = (lds_ptr)smem + ka[0][s];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
        vp[dt] = (lds_ptr)smem + va[dt];

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
        o[dt] = f32x16{};
    float m_used = -INFINITY;
    float l_sum = 0.f;
    const float c = args.scale_log2;

    const int k_end = CAUSAL ? min(Sk, q0 + BM) : Sk;
    const int nb = (k_end + BN - 1) / BN;
    if (nb > 0)
        issue_block(0, 0);
    wait_vmcnt<0>();
    __syncthreads();

    for (int t = 0; t < nb; ++t) {
        // the next block goes into the other stage, last read in block t - 1
        // (before the barrier that ended it)
        if (t + 1 < nb)
            issue_block(t + 1, (t + 1) % STAGES);
        const int kb = t * BN;

        // The block is processed as four 32-key quarters (kt), each through
        // scores, online softmax and the second product, which keeps only one
        // quarter's scores live.
        const bool need_mask = kb + BN > Sk || (CAUSAL && kb + BN - 1 > q0);
        // ---- S^T = K Q^T (32 keys x 32 queries) of quarter kt: the 8 K
        // fragments are requested before the first MFMA, so that the MFMAs
        // do not wait on their reads one by one
        auto scores = [&](int kt) __attribute__((always_inline)) {
            u32x4 kf[8];
#pragma unroll
            for (int s = 0; s < 8; ++s)
                kf[s] = lds_u4_at(kp[s] + 8192 * kt);   // + 32 rows
            __builtin_amdgcn_sched_barrier(0);
            f32x16 sc = f32x16{};
#pragma unroll
            for (int s = 0; s < 8; ++s)
                sc = T::mfma32(kf[s], qf[s], sc);
            return sc;
        };
        // The score MFMAs of quarter kt + 1 are issued before the softmax of
        // quarter kt, so that the matrix unit works on them while the wave's
        // vector ALU does the softmax.
        f32x16 s_next = scores(0);
#pragma unroll
        for (int kt = 0; kt < BN / 32; ++kt) {
            f32x16 sacc = s_next;
            if (kt + 1 < BN / 32)
                s_next = scores(kt + 1);

            // ---- online softmax: score e of the lane is key kb + 32 kt + 8 (e/4) + 4 lh + e%4
            // masking (only in blocks that need it) and the block maximum
            auto mask_max = [&](auto mask_c) __attribute__((always_inline)) {
                constexpr bool MASK = decltype(mask_c)::value;
                // visible if off < Sk - key0 and (causal) off <= qi - key0, with a
                // compile-time off = 8 (e/4) + e%4: one compare against the
                // smaller bound
                const int key0 = kb + 32 * kt + 4 * lh;
                const int tail = Sk - key0;
                const int lim = CAUSAL ? min(tail, qi - key0 + 1) : tail;
                float mx = -INFINITY;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float v = sacc[e];
                    if constexpr (MASK) {
                        const int off = 8 * (e >> 2) + (e & 3);
                        v = off < lim ? v : -INFINITY;
                        sacc[e] = v;
                    }
                    mx = fmaxf(mx, v);
                }
                return mx;
            };
            float mx = need_mask ? mask_max(std::true_type{}) : mask_max(std::false_type{});
            mx = max_of_halves(mx);
            const float m_blk = mx * c;
            // lazy rescaling: move the maximum only when it grew by more than 2^8
            if (__builtin_amdgcn_ballot_w64(m_blk > m_used + RESCALE_LOG2) != 0) {
                const float m_new = fmaxf(m_used, m_blk);
                const float alpha = m_used == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_used - m_new);
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    o[dt] *= alpha;
                l_sum *= alpha;
                m_used = m_new;
            }
            // probabilities rounded to the input format; the running sum adds
            // the rounded values, the same weights the second product uses
            const float m_ref = m_used == -INFINITY ? 0.f : m_used;
            uint32_t pw[8];
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                pw[e / 2] = Prob<T>::pack(__builtin_amdgcn_exp2f(fmaf(sacc[e], c, -m_ref)),
                                          __builtin_amdgcn_exp2f(fmaf(sacc[e + 1], c, -m_ref)));
                l_sum = Prob<T>::add_pair(pw[e / 2], l_sum);
            }
            // key step u = 2 kt + half: the lane's 8 keys are e = 8 half + 0..7
            u32x4 pf[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                pf[hf] = u32x4{pw[4 * hf], pw[4 * hf + 1], pw[4 * hf + 2], pw[4 * hf + 3]};

            // ---- O^T += V^T P^T over the half's two 16-key steps
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int u = 2 * kt + hf;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const u32x2 lo = lds_tr_at(vp[dt] + 4096 * u);          // 16 rows of 256 bytes per step
                    const u32x2 hi = lds_tr_at(vp[dt] + 4096 * u + 2048);   // + 8 rows
                    o[dt] = T::mfma32(u32x4{lo.x, lo.y, hi.x, hi.y}, pf[hf], o[dt]);
                }
            }
        }

        // next block landed (this wave's loads; the barrier covers everyone's),
        // and every wave is done with this stage before it is refilled
        wait_vmcnt<0>();
        {
            const int adv = (t % STAGES == STAGES - 1) ? -(STAGES - 1) * STAGE_BYTES : STAGE_BYTES;
#pragma unroll
            for (int s = 0; s < 8; ++s)
                kp[s] += adv;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                vp[dt] += adv;
        }
        __syncthreads();
    }

    // ---- normalise and store: lane holds O[query][d] for d = 32 dt + 8 (e/4) + 4 lh + e%4
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        args.O, (short)0, (int)((uint32_t)args.B * (uint32_t)Sq * tok), 0x00020000);
    {
        const float l_tot = sum_of_halves(l_sum);
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        const uint32_t base = ((uint32_t)b * (uint32_t)Sq + (uint32_t)qi) * tok + 2u * (uint32_t)h * HD;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint16_t w[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    w[r] = T::from_f32(o[dt][4 * g + r] * inv);
                const uint32_t off = qi < Sq ? base + 2u * (uint32_t)(32 * dt + 8 * g + 4 * lh) : 0xFFFFFFF0u;
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2(w[0], w[1]), pack2(w[2], w[3])}, ro, (int)off,
                                                      0, 0);
            }
    }
}

template <class T>
hipError_t launch_typed(const AttnArgs &a, hipStream_t stream) {
    const int nqb = (a.Sq + BM - 1) / BM;
    if (a.causal)
        hipLaunchKernelGGL((attention_fwd_kernel<T, true>), dim3(nqb * a.H * a.B), dim3(NTHREADS), 0, stream, a);
    else
        hipLaunchKernelGGL((attention_fwd_kernel<T, false>), dim3(nqb * a.H * a.B), dim3(NTHREADS), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_fwd(int dtype, const AttnArgs &a, hipStream_t stream) {
    return dtype == 0 ? launch_typed<F16>(a, stream) : launch_typed<BF16>(a, stream);
}

}  // namespace tg
