// gemm_tiled.hip -- tiled MFMA GEMM for gfx950 (MI355X), direct-load path.
//
// The tiling is the one the TileLang pages teach ("TileLang: writing LLM GPU
// kernels by thinking in tiles", section 2 and the section 3 listing; "TileLang:
// you write the dataflow, the compiler owns the schedule", sections "The tile
// program", "What a tile costs, exactly" and "Software pipelining"): one
// workgroup per output tile, a loop over k-slices that copies an A tile and a B
// tile from global memory into on-chip memory, a tile matrix multiply into a
// register accumulator held in fp32, and one write-back of the tile after the
// loop, with the copies of later slices in flight while the current one is
// multiplied.  Sizes and mechanics are chosen for CDNA4 rather than taken from
// the pages' NVIDIA example:
//
//   * tile 256 x 256, 256 threads = 4 wave64s, each owning a 128 x 128 quarter
//     of C as 4 x 4 v_mfma_f32_32x32x16 accumulators (256 fp32 values per lane,
//     in AGPRs);
//   * k-slices of 32 in a ring of 4 LDS stages (4 x 32 KB of the 160 KB LDS),
//     filled by buffer loads that write LDS directly (buffer_load_dwordx4 ...
//     lds): no staging registers, no LDS store instructions, and each slice is
//     requested two slices before it is used, so a whole slice of MFMA work
//     hides the memory latency twice over; one barrier per slice;
//   * A is staged as [256 m][32 k] (k-contiguous, what a 16-bit MFMA operand
//     holds per lane) and read with ds_read_b128; B stays [32 k][256 n] as in
//     memory and its MFMA fragments come from ds_read_b64_tr_b16, which hands
//     each lane one column of a 4 x 16 block of 16-bit values (lane i of a
//     16-lane group gets element i%4 of the 8 bytes addressed by lane
//     4 j + i/4, for j = 0..3);
//   * XOR swizzles on the 16-byte chunks of both tiles make the fragment
//     reads bank-conflict free; since a direct load writes its 64 lanes' data
//     contiguously, the swizzle is applied to which global chunk each lane
//     fetches;
//   * MFMA fragments are double-buffered in registers: the reads for the next
//     k-step are issued between the MFMAs of the current one;
//   * the MFMA takes the B fragment first, so each lane ends up with 4
//     consecutive output columns of a row, stored with one 8-byte write after
//     the fused bias + GELU(tanh) epilogue (tg_tile.h);
//   * XCD-aware grouped raster of the tiles (tg_tile.h).
//
// The direct loads are issued from inline assembly and their completion is
// awaited with explicit vmcnt waits: the compiler cannot tell that the LDS
// they write is not the LDS being read, and would otherwise wait for every
// load in flight before each use of LDS data.
//
// Rows need not be 16-byte aligned: the direct loads take 2-byte-aligned
// addresses, and the few chunks that then hold wrong data in the last
// k-slice are rewritten before use (fix_last_slice below).
//
// Loads are range-checked buffer loads over each operand's exact byte range;
// an out-of-range lane writes zeros.  k >= K is pushed out of range (offset +
// 2^31) in both A and B, so the K tail is zero on both sides; rows m >= M and
// columns n >= N are never stored, so what they load does not matter.
#include "tg_tile.h"

#include <type_traits>
#include <utility>

namespace tg {
namespace {

using tile::BM;
using tile::BN;
using tile::NTHREADS;
constexpr int BK = 32;
constexpr int STAGES = 4;
constexpr int A_BYTES = BM * BK * 2;              // 16 KB: [256 m][32 k]
constexpr int B_BYTES = BK * BN * 2;              // 16 KB: [32 k][256 n]
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;    // 32 KB
constexpr uint32_t OOB_BUMP = 0x80000000u;        // + offset < 2^31 - 64 KiB -> beyond the operand's buffer

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// A row = 32 k = 4 chunks of 16 B.  A fragment read takes one logical chunk
// from 32 consecutive rows; with this swizzle any 8 consecutive rows of one
// parity and any 16 consecutive rows of one residue mod 4 use 4 different
// slots, which keeps both 32-bank (8 lanes x 16 B) and 64-bank (16 lanes)
// passes conflict free.
__device__ __forceinline__ int a_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// B row = 256 n = 32 chunks.  A transposed read pass touches 4 consecutive
// k-rows (k % 4 = 0..3) and 2 (32-bank pass) or 4 (64-bank pass) adjacent
// chunks; g(k%4) = {0, 10, 4, 14} gives those 4 rows distinct bits 1-2 and
// distinct bits 2-3 of the slot, so every pass hits distinct banks.
__device__ __forceinline__ int b_swz(int k) { return ((k & 1) ? 10 : 0) ^ ((k & 2) ? 4 : 0); }

__device__ __forceinline__ uint32_t lds_address(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

// Buffer resource words for the inline-asm load: base, stride 0, byte range,
// word 3 of the gfx9 family (32-bit data format).
__device__ __forceinline__ i32x4 rsrc_words(const void *base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return i32x4{(int)(uint32_t)p, (int)(uint32_t)(p >> 32), (int)bytes, 0x00020000};
}

// One 16-byte-per-lane buffer load into LDS: lane L reads 16 bytes at byte
// offset voffset + OFF of the buffer and writes them to LDS at m0 + OFF + 16 L
// (the instruction offset moves both addresses).  Loads that share m0 keep
// the wave from rewriting m0 between them, which stalls until the previous
// direct load has taken its value.
template <int OFF>
__device__ __forceinline__ void dma16(const i32x4 &rsrc, uint32_t voffset, uint32_t m0) {
    static_assert(OFF >= 0 && OFF < 4096, "12-bit instruction offset");
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen offset:%3 lds" ::"v"(voffset), "s"(rsrc), "{m0}"(m0),
                 "i"(OFF));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Per-lane addressing of the 8 direct loads that fill one stage.  Wave w,
// lane L, load q = 0..3:
//   A: tile rows 64 w + 16 q + L/4, physical chunk L%4 -> logical chunk
//      c = L%4 ^ a_swz(row) (8 k); destination stage + 4096 w + 1024 q;
//   B: k-rows 8 w + 2 q + L/32, physical chunk L%32 -> logical chunk
//      c = L%32 ^ b_swz(k) (8 n); destination stage + 16 KB + 4096 w + 1024 q.
// The four loads of one operand share m0 (stage + 4096 w, or + 16 KB) and
// reach their destination through the instruction offset 1024 q, which is
// also added to the memory offset; the lane offsets subtract it back.  So
// that they stay non-negative, the buffers start 4 KB before the operands
// (offsets are operand offsets + 4096) and are 4 KB longer.
struct Dma {
    static constexpr uint32_t SHIFT = 4096;
    i32x4 ra, rb;
    uint32_t a_off[4];   // buffer offset of this lane's A chunk for load q, k0 = 0, minus 1024 q
    int a_k;             // first k of the lane's A chunk within the slice
    uint32_t b_off[4];   // buffer offset of this lane's B chunk for load q, k0 = 0, minus 1024 q
    int b_k[4];          // k-row of load q within the slice
    uint32_t b_row;      // bytes per row of B
    uint32_t m0_a, m0_b; // LDS destinations of load q = 0 in stage 0
    int K;

    __device__ __forceinline__ Dma(const GemmArgs &g, int m0, int n0, int wave, int lane, uint32_t lds0) {
        ra = rsrc_words((const char *)g.A - SHIFT, 2u * (uint32_t)g.M * (uint32_t)g.K + SHIFT);
        rb = rsrc_words((const char *)g.B - SHIFT, 2u * (uint32_t)g.K * (uint32_t)g.N + SHIFT);
        K = g.K;
        const int arow = 64 * wave + (lane >> 2);
        const int ac = (lane & 3) ^ a_swz(lane >> 2);
        a_k = 8 * ac;
        b_row = 2u * (uint32_t)g.N;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            a_off[q] = SHIFT - 1024u * q + 2u * ((uint32_t)(m0 + arow + 16 * q) * (uint32_t)g.K + (uint32_t)a_k);
            const int k = 8 * wave + 2 * q + (lane >> 5);
            const int c = (lane & 31) ^ b_swz(k);
            b_k[q] = k;
            b_off[q] = SHIFT - 1024u * q + (uint32_t)k * b_row + 2u * (uint32_t)(n0 + 8 * c);
        }
        m0_a = lds0 + 4096u * (uint32_t)wave;
        m0_b = lds0 + (uint32_t)A_BYTES + 4096u * (uint32_t)wave;
    }

    // Direct load d (0..7) of k-slice kt into LDS stage st: A load d for
    // d < 4, B load d - 4 otherwise.  FULL: the slice lies inside [0, K), so
    // no lane needs the K mask (only the last slice can be partial).
    template <bool FULL, int D>
    __device__ __forceinline__ void issue_one(int kt, int st) const {
        constexpr int q = D & 3;
        const int k0 = kt * BK;
        const uint32_t sbase = (uint32_t)st * (uint32_t)STAGE_BYTES;
        if constexpr (D < 4) {
            uint32_t off = a_off[q] + 2u * (uint32_t)k0;
            if constexpr (!FULL)
                off += (k0 + a_k < K) ? 0u : OOB_BUMP;
            dma16<1024 * q>(ra, off, m0_a + sbase);
        } else {
            uint32_t off = b_off[q] + (uint32_t)k0 * b_row;
            if constexpr (!FULL)
                off += (k0 + b_k[q] < K) ? 0u : OOB_BUMP;
            dma16<1024 * q>(rb, off, m0_b + sbase);
        }
    }

    // Request k-slice kt into LDS stage st.
    __device__ __forceinline__ void issue(int kt, int st) const {
        issue_one<false, 0>(kt, st);
        issue_one<false, 1>(kt, st);
        issue_one<false, 2>(kt, st);
        issue_one<false, 3>(kt, st);
        issue_one<false, 4>(kt, st);
        issue_one<false, 5>(kt, st);
        issue_one<false, 6>(kt, st);
        issue_one<false, 7>(kt, st);
    }
};

// Per-lane LDS byte offsets (within a stage) of the fragment reads of k-step
// s (16 k each):
//   A, ds_read_b128: row wm*128 + 32 i + l%32, logical chunk 2 s + l/32;
//   B, ds_read_b64_tr_b16 twice (k 0..3 and 4..7 of the lane's 8): lane
//      16 G + q addresses k-row 16 s + 8 (G/2) + q/4 (+4), columns
//      wn*128 + 32 j + 16 (G%2) + 4 (q%4) .. +3, so that lane l receives
//      column wn*128 + 32 j + l%32, k = 16 s + 8 (l/32) + 0..7.
struct FragAddr {
    uint32_t a[2][4];    // [s][i]
    uint32_t b[2][4];    // [s][j], first read; the second is +4 rows = +2048 bytes

    __device__ __forceinline__ FragAddr(int wm, int wn, int lane) {
        const int lr = lane & 31;
        const int row0 = wm * 128 + lr;
        const int sw = a_swz(lr);                     // a_swz depends on row bits 1..3 only
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 2 * s + (lane >> 5);
                a[s][i] = 16u * (uint32_t)((row0 + 32 * i) * 4 + (c ^ sw));
            }
        const int G = lane >> 4;
        const int q = lane & 15;
        const int kr = 8 * (G >> 1) + (q >> 2);      // k-row for s = 0, first read; kr % 4 = q / 4
        const int bsw = b_swz(kr);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = wn * 128 + 32 * j + 16 * (G & 1) + 4 * (q & 3);
                const int c = (n >> 3) ^ bsw;
                b[s][j] = (uint32_t)A_BYTES + 512u * (uint32_t)(kr + 16 * s) + 16u * (uint32_t)c +
                          8u * (uint32_t)(q & 1);
            }
    }
};

struct Frag {
    u32x4 a[4], b[4];
};

__device__ __forceinline__ u32x4 lds_u4(uint32_t byte) {
    return *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)byte;
}

__device__ __forceinline__ u32x2 lds_tr(uint32_t byte) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)byte);
    return __builtin_bit_cast(u32x2, v);
}

// Fragment read number r (0..11) of k-step s: r < 4 is A row-block r, then
// B column-block (r-4)/2, first (k 0..3) or second (k 4..7) half.
__device__ __forceinline__ void read_one(Frag &f, const FragAddr &ad, uint32_t stage, int s, int r) {
    if (r < 4) {
        f.a[r] = lds_u4(stage + ad.a[s][r]);
    } else {
        const int j = (r - 4) >> 1;
        if (((r - 4) & 1) == 0) {
            const u32x2 v = lds_tr(stage + ad.b[s][j]);
            f.b[j].x = v.x;
            f.b[j].y = v.y;
        } else {
            const u32x2 v = lds_tr(stage + ad.b[s][j] + 2048u);
            f.b[j].z = v.x;
            f.b[j].w = v.y;
        }
    }
}

// One k-step in a fixed issue order: MFMA q (A block q/4 x B block q%4),
// then fragment read q of the next step (q < 12), then one direct load
// after MFMAs 1, 5, 9, 13 (`dma(d)` for d = 0..3).  sched_barrier keeps the
// compiler from regrouping: spreading the direct loads lets the memory
// pipeline take them while the matrix unit stays busy.
template <class T, bool READ, bool DMA, int Q, typename DmaFn>
__device__ __forceinline__ void kstep_one(const Frag &cur, Frag &nxt, f32x16 (&acc)[4][4], const FragAddr &ad,
                                          uint32_t rstage, int rs, DmaFn &dma) {
    acc[Q >> 2][Q & 3] = T::mfma32(cur.b[Q & 3], cur.a[Q >> 2], acc[Q >> 2][Q & 3]);
    if constexpr (READ && Q < 12)
        read_one(nxt, ad, rstage, rs, Q);
    if constexpr (DMA && (Q & 3) == 1)
        dma(std::integral_constant<int, (Q >> 2)>{});
    __builtin_amdgcn_sched_barrier(0);
}

template <class T, bool READ, bool DMA, typename DmaFn, int... Q>
__device__ __forceinline__ void kstep_seq(const Frag &cur, Frag &nxt, f32x16 (&acc)[4][4], const FragAddr &ad,
                                          uint32_t rstage, int rs, DmaFn &dma, std::integer_sequence<int, Q...>) {
    (kstep_one<T, READ, DMA, Q>(cur, nxt, acc, ad, rstage, rs, dma), ...);
}

template <class T, bool READ, bool DMA, typename DmaFn>
__device__ __forceinline__ void kstep(const Frag &cur, Frag &nxt, f32x16 (&acc)[4][4], const FragAddr &ad,
                                      uint32_t rstage, int rs, DmaFn dma) {
    kstep_seq<T, READ, DMA>(cur, nxt, acc, ad, rstage, rs, dma, std::make_integer_sequence<int, 16>{});
}

// Persistent: the grid has at most one workgroup per CU, and workgroup g
// computes tiles g, g + G, g + 2G, ... (G = grid size, a multiple of the 8
// XCDs when the tile count allows, so every tile of a workgroup stays on its
// XCD in the raster), which removes the dispatch gap between tiles.
// Shapes with K % 8 != 0 or N % 8 != 0 (GEN): the direct loads still move
// 16 bytes per lane, now at 2-byte-aligned addresses, which the hardware
// takes.  Two kinds of chunk in the last k-slice then hold wrong data:
//   * the chunk of each A row that crosses k = K carries the next row's first
//     elements (not zeros) past K, and for the last row of A it crosses the
//     end of the buffer, so the range check zeroes it whole;
//   * the chunk of B's last row that crosses n = N crosses the end of the
//     buffer and is zeroed whole.
// fix_last_slice() rewrites exactly those chunks in LDS from element loads
// (past K or N the loads are out of range and read zero), after the slice's
// direct loads have landed and before the barrier that publishes it.  Each
// chunk is rewritten by a lane of the wave whose direct load wrote it, so
// that wave's own wait orders the two writes.  Chunks of B rows crossing
// n = N elsewhere only feed columns that are never stored.
template <class T>
__device__ __forceinline__ void fix_last_slice(const GemmArgs &g, int m0, int n0, int kl, uint32_t stage) {
    const int k0 = kl * BK;
    const int tid = threadIdx.x;
    if (g.K % 8 != 0) {
        const __amdgpu_buffer_rsrc_t ra = tile::buffer_of(g.A, 2u * (uint32_t)g.M * (uint32_t)g.K);
        const int r = tid;                       // tile row r was loaded by wave r / 64 = this wave
        const int cp = (g.K - k0) >> 3;          // the crossing chunk (< 4: the slice holds K - 1)
        const int v = (g.K - k0) & 7;            // its elements below K
        const uint32_t row = (uint32_t)(m0 + r); // rows >= M read zero (beyond the buffer)
        const uint32_t base = 2u * (row * (uint32_t)g.K + (uint32_t)(k0 + 8 * cp));
        uint16_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            e[q] = q < v ? __builtin_amdgcn_raw_buffer_load_b16(ra, (int)(base + 2u * q), 0, 0) : (uint16_t)0;
        const u32x4 chunk = {pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7])};
        *(__attribute__((address_space(3))) u32x4 *)(uintptr_t)(stage + 64u * r + 16u * (cp ^ a_swz(r))) = chunk;
    }
    if (g.N % 8 != 0 && n0 <= g.N - 1 && g.N - 1 < n0 + BN) {
        const int r = g.K - 1 - k0;              // B's last row, loaded by wave r / 8
        if (tid == 64 * (r >> 3)) {
            const __amdgpu_buffer_rsrc_t rb = tile::buffer_of(g.B, 2u * (uint32_t)g.K * (uint32_t)g.N);
            const int c = (g.N - 1 - n0) >> 3;
            const uint32_t base = 2u * ((uint32_t)(g.K - 1) * (uint32_t)g.N + (uint32_t)(n0 + 8 * c));
            uint16_t e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                e[q] = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)(base + 2u * q), 0, 0);
            const u32x4 chunk = {pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7])};
            *(__attribute__((address_space(3))) u32x4 *)(uintptr_t)(stage + (uint32_t)A_BYTES + 512u * r +
                                                                    16u * (c ^ b_swz(r))) = chunk;
        }
    }
}

// Epilogue and store through LDS.  After the k-loop the 128 KiB stage ring
// is free and holds the whole 256 x 256 C tile of 16-bit values (512-byte
// rows).  Each lane applies the epilogue to its accumulators and writes its
// 4-column groups to LDS (16-byte chunk index XOR row % 32: the 32 rows one
// instruction touches land on different chunks); then every wave copies whole
// rows out, 16 bytes per lane, 2 rows of 512 bytes per instruction, so HBM
// sees full row segments instead of 16-byte pieces of 32 rows (which, at
// 2-byte-aligned row starts, split across write sectors).  Chunks that cross
// column N go out element by element.  The caller's barrier after this keeps
// the next tile's loads from overwriting LDS before every wave has read it.
template <class T, int EPI, bool ALIGNED>
__device__ __forceinline__ void store_tile_lds(const GemmArgs &args, const f32x16 (&acc)[4][4], int m0, int n0,
                                               int wm, int wn, int lane, uint32_t lds0) {
    const int M = args.M, N = args.N;
    const int lr = lane & 31;
    const int lh = lane >> 5;
    // The bias of all 16 four-column groups of this lane, requested at once
    // (range-checked: columns past N read zero), before the barrier.
    uint32_t braw[4][4][2];
    if constexpr (EPI != EPI_NONE) {
        const __amdgpu_buffer_rsrc_t rb = tile::buffer_of(args.bias, 2u * (uint32_t)N);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t off = 2u * (uint32_t)(n0 + wn * 128 + 32 * j + 8 * q + 4 * lh);
                if constexpr (ALIGNED) {   // N % 8 == 0: a group is all inside or all outside
                    const u32x2 raw = __builtin_amdgcn_raw_buffer_load_b64(rb, (int)off, 0, 0);
                    braw[j][q][0] = raw.x;
                    braw[j][q][1] = raw.y;
                } else {
                    uint16_t e[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        e[r] = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)(off + 2u * r), 0, 0);
                    braw[j][q][0] = pack2(e[0], e[1]);
                    braw[j][q][1] = pack2(e[2], e[3]);
                }
            }
    }
    __syncthreads();   // every wave is done reading the last slice
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int col = wn * 128 + 32 * j + 8 * q + 4 * lh;
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (EPI != EPI_NONE) {
                bv[0] = T::to_f32((uint16_t)(braw[j][q][0] & 0xffff));
                bv[1] = T::to_f32((uint16_t)(braw[j][q][0] >> 16));
                bv[2] = T::to_f32((uint16_t)(braw[j][q][1] & 0xffff));
                bv[3] = T::to_f32((uint16_t)(braw[j][q][1] >> 16));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm * 128 + 32 * i + lr;
                uint16_t o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[r] = T::from_f32(epilogue<EPI>(acc[i][j][4 * q + r], bv[r]));
                const uint32_t chunk = (uint32_t)(col >> 3) ^ (uint32_t)(row & 31);
                const uint32_t addr = lds0 + 512u * (uint32_t)row + 16u * chunk + 8u * (uint32_t)lh;
                *(__attribute__((address_space(3))) u32x2 *)(uintptr_t)addr =
                    u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
            }
        }
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rc = tile::buffer_of(args.C, 2u * (uint32_t)M * (uint32_t)N);
    const int tid = threadIdx.x;
#pragma unroll 4
    for (int it = 0; it < 32; ++it) {
        const int idx = it * NTHREADS + tid;
        const int row = idx >> 5;
        const int c = idx & 31;
        const int m = m0 + row;
        const int n = n0 + 8 * c;
        const u32x4 v = *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)(
            lds0 + 512u * (uint32_t)row + 16u * (uint32_t)(c ^ (row & 31)));
        const uint32_t base = 2u * ((uint32_t)m * (uint32_t)N + (uint32_t)n);
        if (ALIGNED || n + 8 <= N) {
            const uint32_t off = (m < M && n < N) ? base : tile::OOB;
            __builtin_amdgcn_raw_buffer_store_b128(v, rc, (int)off, 0, 0);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t off = (m < M && n + e < N) ? base + 2u * e : tile::OOB;
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(v[e >> 1] >> (16 * (e & 1))), rc, (int)off, 0, 0);
            }
        }
    }
}

template <class T, int EPI, bool GEN>
__global__ __launch_bounds__(NTHREADS) void gemm_tiled_kernel(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) u32x4 smem[STAGES * STAGE_BYTES / 16];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const uint32_t lds0 = lds_address(smem);
    auto stage = [&](int st) { return lds0 + (uint32_t)st * (uint32_t)STAGE_BYTES; };
    const int total = ((args.M + BM - 1) / BM) * ((args.N + BN - 1) / BN);
    const int nk = (args.K + BK - 1) / BK;

    for (int w = blockIdx.x; w < total; w += gridDim.x) {
        // The lane id is made opaque per tile so that the per-lane addresses
        // below are recomputed for each tile instead of being hoisted out of
        // the tile loop, where they would stay live through the k-loop.
        int lane = threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        const FragAddr fad(wm, wn, lane);
        int tm, tn;
        tile::tile_of_workgroup(args.M, args.N, w, tm, tn);
        const int m0 = tm * BM;
        const int n0 = tn * BN;
        const Dma dma(args, m0, n0, wave, lane, lds0);

        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = f32x16{};

        Frag f0, f1;
        // Prologue: request slices 0..2, wait for slice 0.  The previous
        // tile's C stores are older than these loads, so the same counts hold.
        if (nk > 0) {
            dma.issue(0, 0);
            if (nk > 1)
                dma.issue(1, 1);
            if (nk > 2) {
                dma.issue(2, 2);
                wait_vmcnt<16>();
            } else if (nk > 1) {
                wait_vmcnt<8>();
            } else {
                wait_vmcnt<0>();
                if constexpr (GEN)
                    fix_last_slice<T>(args, m0, n0, 0, stage(0));
            }
        }
        __syncthreads();
        if (nk > 0) {
#pragma unroll
            for (int r = 0; r < 12; ++r)
                read_one(f0, fad, stage(0), 0, r);
        }

        // Slice t in stage t%4, fragments of its first k-step already in f0:
        //   step 0: MFMAs on f0, reads of step 1 into f1, first half of the
        //           direct loads of slice t+3 into stage (t+3)%4 (that stage was
        //           last read in slice t-1, before the previous barrier);
        //   wait until this wave's loads of slice t+1 have landed, barrier
        //           (everyone's have, and everyone's reads of slice t are done);
        //   step 1: MFMAs on f1, reads of step 0 of slice t+1 into f0, second
        //           half of the direct loads of slice t+3.
        // Loads issued after slice t+1's when waiting: all 8 of slice t+2 and
        // the first 4 of slice t+3, hence vmcnt(12) in the steady state.
        // ISSUE: 0 = no loads, 1 = loads of a full slice, 2 = loads of the
        // (possibly partial) last slice.
        auto slice = [&](int t, auto issue, auto wait, auto next) __attribute__((always_inline)) {
            const uint32_t st = stage(t & 3);
            constexpr int ISSUE_KIND = decltype(issue)::value;
            constexpr bool ISSUE = ISSUE_KIND != 0;
            constexpr bool FULL = ISSUE_KIND == 1;
            constexpr bool NEXT = decltype(next)::value;
            const int kt = t + 3;
            auto dma_lo = [&](auto d) __attribute__((always_inline)) {
                dma.template issue_one<FULL, decltype(d)::value>(kt, kt & 3);
            };
            auto dma_hi = [&](auto d) __attribute__((always_inline)) {
                dma.template issue_one<FULL, decltype(d)::value + 4>(kt, kt & 3);
            };
            kstep<T, true, ISSUE>(f0, f1, acc, fad, st, 1, dma_lo);
            if constexpr (NEXT) {
                wait_vmcnt<decltype(wait)::value>();
                // with nothing left in flight, slice t + 1 is the last one
                if constexpr (GEN && decltype(wait)::value == 0)
                    fix_last_slice<T>(args, m0, n0, t + 1, stage((t + 1) & 3));
                __syncthreads();
            }
            kstep<T, NEXT, ISSUE>(f1, f0, acc, fad, stage((t + 1) & 3), 0, dma_hi);
        };
        using yes = std::true_type;
        using no = std::false_type;
        using none = std::integral_constant<int, 0>;
        using full = std::integral_constant<int, 1>;
        using last = std::integral_constant<int, 2>;
        using w12 = std::integral_constant<int, 12>;
        using w8 = std::integral_constant<int, 8>;
        using w0 = std::integral_constant<int, 0>;
        int t = 0;
        for (; t + 4 < nk; ++t)
            slice(t, full{}, w12{}, yes{});
        if (t + 3 < nk) {
            slice(t, last{}, w12{}, yes{});
            ++t;
        }
        if (t + 3 == nk && t < nk) {
            slice(t, none{}, w8{}, yes{});
            ++t;
        }
        if (t + 2 == nk && t < nk) {
            slice(t, none{}, w0{}, yes{});
            ++t;
        }
        if (t + 1 == nk)
            slice(t, none{}, w0{}, no{});

        store_tile_lds<T, EPI, !GEN>(args, acc, m0, n0, wm, wn, lane, lds0);
        // every wave is done reading LDS before the next tile's loads land
        __syncthreads();
    }
}

template <class T, int EPI>
hipError_t launch_typed(const GemmArgs &a, bool gen, int grid, hipStream_t stream) {
    if (gen)
        hipLaunchKernelGGL((gemm_tiled_kernel<T, EPI, true>), dim3(grid), dim3(NTHREADS), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_tiled_kernel<T, EPI, false>), dim3(grid), dim3(NTHREADS), 0, stream, a);
    return hipGetLastError();
}

template <class T>
hipError_t launch_epi(int epi, const GemmArgs &a, bool gen, int grid, hipStream_t stream) {
    switch (epi) {
    case EPI_NONE: return launch_typed<T, EPI_NONE>(a, gen, grid, stream);
    case EPI_BIAS: return launch_typed<T, EPI_BIAS>(a, gen, grid, stream);
    default: return launch_typed<T, EPI_BIAS_GELU_TANH>(a, gen, grid, stream);
    }
}

}  // namespace

hipError_t launch_tiled_vec(int dtype, int epi, const GemmArgs &a, bool aligned, int num_cu, hipStream_t stream) {
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    int grid = tiles;
    if (num_cu > 0 && tiles > num_cu) {
        // one workgroup per CU, rounded down to a multiple of the XCD count
        grid = num_cu >= tile::NUM_XCD ? num_cu - num_cu % tile::NUM_XCD : num_cu;
    }
    return dtype == 0 ? launch_epi<F16>(epi, a, !aligned, grid, stream)
                      : launch_epi<BF16>(epi, a, !aligned, grid, stream);
}

}  // namespace tg
