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
//   * tile BM x BN with BM, BN in {128, 256} (the tile configuration is a
//     template parameter; the host picks one per shape), 256 threads = 4
//     wave64s in a 2 x 2 grid, each owning a BM/2 x BN/2 block of C as
//     v_mfma_f32_32x32x16 accumulators in AGPRs (256 fp32 values per lane at
//     256 x 256);
//   * k-slices of 32 in a ring of 4 LDS stages (4 x 32 KB of the 160 KB LDS at
//     256 x 256), filled by buffer loads that write LDS directly
//     (buffer_load_dwordx4 ... lds): no staging registers, no LDS store
//     instructions, and each slice is requested two slices before it is used,
//     so a whole slice of MFMA work hides the memory latency twice over; one
//     barrier per slice;
//   * A is staged as [BM m][32 k] (k-contiguous, what a 16-bit MFMA operand
//     holds per lane) and read with ds_read_b128; B stays [32 k][BN n] as in
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
//     consecutive output columns of a row; after the fused bias + GELU(tanh)
//     epilogue each wave's block of C goes through LDS 32 rows at a time
//     and leaves as row segments;
//   * persistent grid with an XCD-aware grouped raster of the tiles
//     (tg_tile.h); the smaller tiles fit two workgroups per CU.
//
// The direct loads (tg_direct.h) are issued from inline assembly and their
// completion is awaited with explicit vmcnt waits.
//
// Rows need not be 16-byte aligned: the direct loads take 2-byte-aligned
// addresses, and the few chunks that then hold wrong data in the last
// k-slice are rewritten before use (fix_last_slice below).
//
// Loads are range-checked buffer loads over each operand's exact byte range;
// an out-of-range lane writes zeros.  k >= K is pushed out of range (offset +
// 2^31) in both A and B, so the K tail is zero on both sides; rows m >= M and
// columns n >= N are never stored, so what they load does not matter.
#include "tg_direct.h"
#include "tg_tile.h"

#include <type_traits>
#include <utility>

namespace tg {
namespace {

using tile::NTHREADS;
using namespace direct;
constexpr int BK = 32;
constexpr int STAGES = 4;
constexpr uint32_t OOB_BUMP = 0x80000000u;        // + offset < 2^31 - 64 KiB -> beyond the operand's buffer

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Everything that follows from the tile size.  Waves form a 2 x 2 grid over
// the tile; each owns WM x WN = (BM/2) x (BN/2) of C as I x J accumulators
// of 32 x 32.  Per k-slice and wave: QA direct loads of A (16 rows of 64
// bytes each) and QB of B (1 KB = RB k-rows each).
template <int BM_, int BN_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_;
    static_assert((BM == 128 || BM == 256) && (BN == 128 || BN == 256), "tile sizes");
    static constexpr int WM = BM / 2, WN = BN / 2;
    static constexpr int I = WM / 32, J = WN / 32;
    static constexpr int A_BYTES = BM * BK * 2;             // [BM m][32 k]
    static constexpr int B_BYTES = BK * BN * 2;             // [32 k][BN n]
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int B_ROW = 2 * BN;                    // bytes per k-row of the B stage
    static constexpr int CPR = BN / 8;                      // 16-byte chunks per B row (and per C row)
    static constexpr int QA = BM / 64, QB = BN / 64;
    static constexpr int D = QA + QB;                       // direct loads per slice per wave
    static constexpr int RB = 512 / BN;                     // B k-rows per direct load
    static constexpr int A_ROWS_PER_WAVE = BM / 4;
    static constexpr int READS = I + 2 * J;                 // fragment reads per k-step
    static constexpr int MFMAS = I * J;                     // MFMAs per k-step
    static constexpr int OCCUPANCY = (STAGES * STAGE_BYTES <= 80 * 1024) ? 2 : 1;   // workgroups per CU
    static_assert(D % 2 == 0, "loads split over the two k-steps of a slice");
};

// A row = 32 k = 4 chunks of 16 B.  A fragment read takes one logical chunk
// from 32 consecutive rows; with this swizzle any 8 consecutive rows of one
// parity and any 16 consecutive rows of one residue mod 4 use 4 different
// slots, which keeps both 32-bank (8 lanes x 16 B) and 64-bank (16 lanes)
// passes conflict free.
__device__ __forceinline__ int a_swz(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// B row = BN n = 32 or 16 chunks.  A transposed read pass touches 4
// consecutive k-rows (k % 4 = 0..3) and 2 (32-bank pass) or 4 (64-bank pass)
// adjacent chunks; g(k%4) = {0, 10, 4, 14} gives those 4 rows distinct bits
// 1-2 and distinct bits 2-3 of the slot, so every pass hits distinct banks
// (the 64 banks span 256 bytes, so only the chunk index mod 16 matters).
__device__ __forceinline__ int b_swz(int k) { return ((k & 1) ? 10 : 0) ^ ((k & 2) ? 4 : 0); }

// Per-lane addressing of the D direct loads that fill one stage.  Wave w,
// lane L:
//   A load q < QA: tile rows BM/4 w + 16 q + L/4, physical chunk L%4 ->
//      logical chunk c = L%4 ^ a_swz(row) (8 k); destination
//      stage + 16 BM w + 1024 q;
//   B load q < QB: k-row 8 w + RB q + L/CPR, physical chunk L%CPR ->
//      logical chunk c = L%CPR ^ b_swz(k) (8 n); destination
//      stage + A_BYTES + 16 BN w + 1024 q.
// The loads of one operand share m0 (their q = 0 destination) and reach
// their destination through the instruction offset 1024 q, which is also
// added to the memory offset; the lane offsets subtract it back.  So that
// they stay non-negative, the buffers start 4 KB before the operands
// (offsets are operand offsets + 4096) and are 4 KB longer.
template <class C>
struct Dma {
    static constexpr uint32_t SHIFT = 4096;
    i32x4 ra, rb;
    uint32_t a_off[C::QA];   // buffer offset of this lane's A chunk for load q, k0 = 0, minus 1024 q
    int a_k;                 // first k of the lane's A chunk within the slice
    uint32_t b_off[C::QB];   // buffer offset of this lane's B chunk for load q, k0 = 0, minus 1024 q
    int b_k[C::QB];          // k-row of load q within the slice
    uint32_t b_row;          // bytes per row of B
    uint32_t m0_a, m0_b;     // LDS destinations of load q = 0 in stage 0
    int K;

    __device__ __forceinline__ Dma(const GemmArgs &g, int m0, int n0, int wave, int lane, uint32_t lds0) {
        ra = rsrc_words((const char *)g.A - SHIFT, 2u * (uint32_t)g.M * (uint32_t)g.K + SHIFT);
        rb = rsrc_words((const char *)g.B - SHIFT, 2u * (uint32_t)g.K * (uint32_t)g.N + SHIFT);
        K = g.K;
        const int arow = C::A_ROWS_PER_WAVE * wave + (lane >> 2);
        const int ac = (lane & 3) ^ a_swz(lane >> 2);
        a_k = 8 * ac;
        b_row = 2u * (uint32_t)g.N;
#pragma unroll
        for (int q = 0; q < C::QA; ++q)
            a_off[q] = SHIFT - 1024u * q + 2u * ((uint32_t)(m0 + arow + 16 * q) * (uint32_t)g.K + (uint32_t)a_k);
#pragma unroll
        for (int q = 0; q < C::QB; ++q) {
            const int k = 8 * wave + C::RB * q + (int)((unsigned)lane / C::CPR);
            const int c = (int)((unsigned)lane % C::CPR) ^ b_swz(k);
            b_k[q] = k;
            b_off[q] = SHIFT - 1024u * q + (uint32_t)k * b_row + 2u * (uint32_t)(n0 + 8 * c);
        }
        m0_a = lds0 + 16u * C::BM * (uint32_t)wave;
        m0_b = lds0 + (uint32_t)C::A_BYTES + 16u * C::BN * (uint32_t)wave;
    }

    // Direct load d (0..D-1) of k-slice kt into LDS stage st: A load d for
    // d < QA, B load d - QA otherwise.  FULL: the slice lies inside [0, K), so
    // no lane needs the K mask (only the last slice can be partial).
    template <bool FULL, int DI>
    __device__ __forceinline__ void issue_one(int kt, int st) const {
        const int k0 = kt * BK;
        const uint32_t sbase = (uint32_t)st * (uint32_t)C::STAGE_BYTES;
        if constexpr (DI < C::QA) {
            constexpr int q = DI;
            uint32_t off = a_off[q] + 2u * (uint32_t)k0;
            if constexpr (!FULL)
                off += (k0 + a_k < K) ? 0u : OOB_BUMP;
            dma16<1024 * q>(ra, off, m0_a + sbase);
        } else {
            constexpr int q = DI - C::QA;
            uint32_t off = b_off[q] + (uint32_t)k0 * b_row;
            if constexpr (!FULL)
                off += (k0 + b_k[q] < K) ? 0u : OOB_BUMP;
            dma16<1024 * q>(rb, off, m0_b + sbase);
        }
    }

    template <int... DI>
    __device__ __forceinline__ void issue_seq(int kt, int st, std::integer_sequence<int, DI...>) const {
        (issue_one<false, DI>(kt, st), ...);
    }

    // Request k-slice kt into LDS stage st.
    __device__ __forceinline__ void issue(int kt, int st) const {
        issue_seq(kt, st, std::make_integer_sequence<int, C::D>{});
    }
};

// Per-lane LDS byte offsets (within a stage) of the fragment reads of k-step
// s (16 k each):
//   A, ds_read_b128: row wm*WM + 32 i + l%32, logical chunk 2 s + l/32;
//   B, ds_read_b64_tr_b16 twice (k 0..3 and 4..7 of the lane's 8): lane
//      16 G + q addresses k-row 16 s + 8 (G/2) + q/4 (+4), columns
//      wn*WN + 32 j + 16 (G%2) + 4 (q%4) .. +3, so that lane l receives
//      column wn*WN + 32 j + l%32, k = 16 s + 8 (l/32) + 0..7.
template <class C>
struct FragAddr {
    uint32_t a[2][C::I];    // [s][i]
    uint32_t b[2][C::J];    // [s][j], first read; the second is +4 rows

    __device__ __forceinline__ FragAddr(int wm, int wn, int lane) {
        const int lr = lane & 31;
        const int row0 = wm * C::WM + lr;
        const int sw = a_swz(lr);                     // a_swz depends on row bits 1..3 only
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < C::I; ++i) {
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
            for (int j = 0; j < C::J; ++j) {
                const int n = wn * C::WN + 32 * j + 16 * (G & 1) + 4 * (q & 3);
                const int c = (n >> 3) ^ bsw;
                b[s][j] = (uint32_t)C::A_BYTES + (uint32_t)C::B_ROW * (uint32_t)(kr + 16 * s) + 16u * (uint32_t)c +
                          8u * (uint32_t)(q & 1);
            }
    }
};

template <class C>
struct Frag {
    u32x4 a[C::I], b[C::J];
};

__device__ __forceinline__ u32x4 lds_u4(uint32_t byte) {
    return *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)byte;
}

__device__ __forceinline__ u32x2 lds_tr(uint32_t byte) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)byte);
    return __builtin_bit_cast(u32x2, v);
}

// Fragment read number r (0..READS-1) of k-step s: r < I is A row-block r,
// then B column-block (r-I)/2, first (k 0..3) or second (k 4..7) half.
template <class C>
__device__ __forceinline__ void read_one(Frag<C> &f, const FragAddr<C> &ad, uint32_t stage, int s, int r) {
    if (r < C::I) {
        f.a[r] = lds_u4(stage + ad.a[s][r]);
    } else {
        const int j = (r - C::I) >> 1;
        if (((r - C::I) & 1) == 0) {
            const u32x2 v = lds_tr(stage + ad.b[s][j]);
            f.b[j].x = v.x;
            f.b[j].y = v.y;
        } else {
            const u32x2 v = lds_tr(stage + ad.b[s][j] + 4u * (uint32_t)C::B_ROW);
            f.b[j].z = v.x;
            f.b[j].w = v.y;
        }
    }
}

// Fragment reads issued after MFMA Q of a k-step: one each while there are
// at least as many MFMAs as reads, else Q*R/M .. (Q+1)*R/M - 1.
template <class C, int Q>
struct ReadsAfter {
    static constexpr int LO = C::READS <= C::MFMAS ? Q : Q * C::READS / C::MFMAS;
    static constexpr int HI = C::READS <= C::MFMAS ? (Q < C::READS ? Q + 1 : Q) : (Q + 1) * C::READS / C::MFMAS;
};

// Direct load p (0..D/2-1) of a k-step's half goes after MFMA p*M/(D/2) + 1
// (M >= 4 MFMAs per k-step, so that stays below M).
template <class C, int Q>
struct DmaAfter {
    static constexpr int H = C::D / 2;
    static constexpr int find(int p) { return p >= H ? -1 : ((p * C::MFMAS) / H + 1 == Q ? p : find(p + 1)); }
    static constexpr int P = find(0);
};

template <class C, int R0, int... R>
__device__ __forceinline__ void read_range(Frag<C> &nxt, const FragAddr<C> &ad, uint32_t rstage, int rs,
                                           std::integer_sequence<int, R...>) {
    (read_one<C>(nxt, ad, rstage, rs, R0 + R), ...);
}

// One k-step in a fixed issue order: MFMA Q (A block Q/J x B block Q%J),
// then the fragment reads of the next step that follow it, then at most one
// direct load (`dma(p)` for p = 0..D/2-1).  sched_barrier keeps the compiler
// from regrouping: spreading the direct loads lets the memory pipeline take
// them while the matrix unit stays busy.
template <class C, class T, bool READ, bool DMA, int Q, typename DmaFn>
__device__ __forceinline__ void kstep_one(const Frag<C> &cur, Frag<C> &nxt, f32x16 (&acc)[C::I][C::J],
                                          const FragAddr<C> &ad, uint32_t rstage, int rs, DmaFn &dma) {
    acc[Q / C::J][Q % C::J] = T::mfma32(cur.b[Q % C::J], cur.a[Q / C::J], acc[Q / C::J][Q % C::J]);
    if constexpr (READ) {
        constexpr int LO = ReadsAfter<C, Q>::LO, HI = ReadsAfter<C, Q>::HI;
        if constexpr (HI > LO)
            read_range<C, LO>(nxt, ad, rstage, rs, std::make_integer_sequence<int, HI - LO>{});
    }
    if constexpr (DMA && DmaAfter<C, Q>::P >= 0)
        dma(std::integral_constant<int, DmaAfter<C, Q>::P>{});
    __builtin_amdgcn_sched_barrier(0);
}

template <class C, class T, bool READ, bool DMA, typename DmaFn, int... Q>
__device__ __forceinline__ void kstep_seq(const Frag<C> &cur, Frag<C> &nxt, f32x16 (&acc)[C::I][C::J],
                                          const FragAddr<C> &ad, uint32_t rstage, int rs, DmaFn &dma,
                                          std::integer_sequence<int, Q...>) {
    (kstep_one<C, T, READ, DMA, Q>(cur, nxt, acc, ad, rstage, rs, dma), ...);
}

template <class C, class T, bool READ, bool DMA, typename DmaFn>
__device__ __forceinline__ void kstep(const Frag<C> &cur, Frag<C> &nxt, f32x16 (&acc)[C::I][C::J],
                                      const FragAddr<C> &ad, uint32_t rstage, int rs, DmaFn dma) {
    kstep_seq<C, T, READ, DMA>(cur, nxt, acc, ad, rstage, rs, dma, std::make_integer_sequence<int, C::MFMAS>{});
}

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
template <class C, class T>
__device__ __forceinline__ void fix_last_slice(const GemmArgs &g, int m0, int n0, int kl, uint32_t stage) {
    const int k0 = kl * BK;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    if (g.K % 8 != 0 && lane < C::A_ROWS_PER_WAVE) {
        const __amdgpu_buffer_rsrc_t ra = tile::buffer_of(g.A, 2u * (uint32_t)g.M * (uint32_t)g.K);
        const int r = C::A_ROWS_PER_WAVE * wave + lane;   // tile row r was loaded by this wave
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
    if (g.N % 8 != 0 && n0 <= g.N - 1 && g.N - 1 < n0 + C::BN) {
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
            *(__attribute__((address_space(3))) u32x4 *)(uintptr_t)(stage + (uint32_t)C::A_BYTES +
                                                                    (uint32_t)C::B_ROW * r +
                                                                    16u * (c ^ b_swz(r))) = chunk;
        }
    }
}

// Epilogue and store through LDS, one wave at a time.  Each wave takes its
// WM x WN block of C 32 rows (one accumulator row block i) at a time: the
// lanes apply the epilogue to their accumulators and write their 4-column
// groups (8 bytes) to the wave's own LDS buffer of 32 rows x WN 16-bit
// values (chunk index XOR a row swizzle), then the wave reads the rows back
// 16 bytes per lane and stores them, 2 WN contiguous bytes per row, so HBM
// sees row segments instead of 16-byte pieces of 32 rows (which, at
// 2-byte-aligned row starts, split across write sectors); chunks that cross
// column N go out element by element.  The buffers lie in stages the k-loop
// is done with in every wave -- not the stage of the last slice, which a
// slower wave may still be reading -- so no barrier is needed, and LDS
// processes one wave's accesses in order, so a buffer is rewritten only
// after its previous rows were read.  The epilogue arithmetic of one row
// block overlaps the stores of the previous one.  The caller's barrier
// after this keeps the next tile's loads out of the buffers until every
// wave has read its rows.
template <class C>
struct WaveStage {
    static constexpr int CPRW = C::WN / 8;                     // 16-byte chunks per buffer row
    static constexpr int BUF = 32 * C::WN * 2;                 // bytes per wave: 32 rows x WN
    static constexpr int PER_STAGE = C::STAGE_BYTES / BUF;     // buffers per stage
    static_assert(PER_STAGE >= 2 && (4 + PER_STAGE - 1) / PER_STAGE <= 3, "wave buffers fit 3 stages");
    static __device__ __forceinline__ uint32_t swz(int row) {
        return (uint32_t)((row ^ (row / CPRW)) & (CPRW - 1));
    }
};

template <class C, class T, int EPI, bool ALIGNED>
__device__ __forceinline__ void store_tile_wave(const GemmArgs &args, const f32x16 (&acc)[C::I][C::J], int m0,
                                                int n0, int wm, int wn, int wave, int lane, uint32_t lds0,
                                                int nk) {
    using W = WaveStage<C>;
    const int M = args.M, N = args.N;
    const int lr = lane & 31;
    const int lh = lane >> 5;
    // the stage of the last slice is (nk - 1) & 3; the next ones are free
    const uint32_t buf = lds0 + (uint32_t)(((nk + wave / W::PER_STAGE) & 3) * C::STAGE_BYTES) +
                         (uint32_t)((wave % W::PER_STAGE) * W::BUF);
    // The bias of all J four-column groups of this lane, requested at once
    // (range-checked: columns past N read zero).
    uint32_t braw[C::J][4][2];
    if constexpr (EPI != EPI_NONE) {
        const __amdgpu_buffer_rsrc_t rb = tile::buffer_of(args.bias, 2u * (uint32_t)N);
#pragma unroll
        for (int j = 0; j < C::J; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t off = 2u * (uint32_t)(n0 + wn * C::WN + 32 * j + 8 * q + 4 * lh);
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
    const __amdgpu_buffer_rsrc_t rc = tile::buffer_of(args.C, 2u * (uint32_t)M * (uint32_t)N);
#pragma unroll
    for (int i = 0; i < C::I; ++i) {
#pragma unroll
        for (int j = 0; j < C::J; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float bv[4] = {0.f, 0.f, 0.f, 0.f};
                if constexpr (EPI != EPI_NONE) {
                    bv[0] = T::to_f32((uint16_t)(braw[j][q][0] & 0xffff));
                    bv[1] = T::to_f32((uint16_t)(braw[j][q][0] >> 16));
                    bv[2] = T::to_f32((uint16_t)(braw[j][q][1] & 0xffff));
                    bv[3] = T::to_f32((uint16_t)(braw[j][q][1] >> 16));
                }
                uint16_t o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    o[r] = T::from_f32(epilogue<EPI>(acc[i][j][4 * q + r], bv[r]));
                const uint32_t chunk = (uint32_t)(4 * j + q) ^ W::swz(lr);
                *(__attribute__((address_space(3))) u32x2 *)(uintptr_t)(
                    buf + (uint32_t)(2 * C::WN * lr) + 16u * chunk + 8u * (uint32_t)lh) =
                    u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
            }
        }
        // rows wm*WM + 32 i + 0..31 of the tile, columns wn*WN ..: 64 / CPRW
        // rows per read
#pragma unroll
        for (int it = 0; it < 32 * W::CPRW / 64; ++it) {
            const int row = it * (64 / W::CPRW) + lane / W::CPRW;
            const int c = lane % W::CPRW;
            const int m = m0 + wm * C::WM + 32 * i + row;
            const int n = n0 + wn * C::WN + 8 * c;
            const u32x4 v = *(__attribute__((address_space(3))) const u32x4 *)(uintptr_t)(
                buf + (uint32_t)(2 * C::WN * row) + 16u * ((uint32_t)c ^ W::swz(row)));
            const uint32_t base = 2u * ((uint32_t)m * (uint32_t)N + (uint32_t)n);
            if (ALIGNED || n + 8 <= N) {
                const uint32_t off = (m < M && n < N) ? base : tile::OOB;
                __builtin_amdgcn_raw_buffer_store_b128(v, rc, (int)off, 0, 0);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t off = (m < M && n + e < N) ? base + 2u * e : tile::OOB;
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(v[e >> 1] >> (16 * (e & 1))), rc, (int)off, 0,
                                                          0);
                }
            }
        }
    }
}

// Persistent: the grid has at most OCCUPANCY workgroups per CU, and
// workgroup g computes tiles g, g + G, g + 2G, ... (G = grid size, a
// multiple of the 8 XCDs when the tile count allows, so every tile of a
// workgroup stays on its XCD in the raster), which removes the dispatch gap
// between tiles.
template <class C, class T, int EPI, bool GEN>
__global__ __launch_bounds__(NTHREADS, C::OCCUPANCY) void gemm_tiled_kernel(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) u32x4 smem[STAGES * C::STAGE_BYTES / 16];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const uint32_t lds0 = lds_address(smem);
    auto stage = [&](int st) { return lds0 + (uint32_t)st * (uint32_t)C::STAGE_BYTES; };
    const int tiles_m = (args.M + C::BM - 1) / C::BM;
    const int tiles_n = (args.N + C::BN - 1) / C::BN;
    const int total = tiles_m * tiles_n;
    const int nk = (args.K + BK - 1) / BK;
    constexpr int D = C::D;

    for (int w = blockIdx.x; w < total; w += gridDim.x) {
        // The lane id is made opaque per tile so that the per-lane addresses
        // below are recomputed for each tile instead of being hoisted out of
        // the tile loop, where they would stay live through the k-loop.
        int lane = threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        const FragAddr<C> fad(wm, wn, lane);
        int tm, tn;
        tile::tile_of_index(tiles_m, tiles_n, w, tm, tn);
        const int m0 = tm * C::BM;
        const int n0 = tn * C::BN;
        const Dma<C> dma(args, m0, n0, wave, lane, lds0);

        f32x16 acc[C::I][C::J];
#pragma unroll
        for (int i = 0; i < C::I; ++i)
#pragma unroll
            for (int j = 0; j < C::J; ++j)
                acc[i][j] = f32x16{};

        Frag<C> f0, f1;
        // Prologue: request slices 0..2, wait for slice 0.  The previous
        // tile's C stores are older than these loads, so the same counts hold.
        if (nk > 0) {
            dma.issue(0, 0);
            if (nk > 1)
                dma.issue(1, 1);
            if (nk > 2) {
                dma.issue(2, 2);
                wait_vmcnt<2 * D>();
            } else if (nk > 1) {
                wait_vmcnt<D>();
            } else {
                wait_vmcnt<0>();
                if constexpr (GEN)
                    fix_last_slice<C, T>(args, m0, n0, 0, stage(0));
            }
        }
        __syncthreads();
        if (nk > 0) {
#pragma unroll
            for (int r = 0; r < C::READS; ++r)
                read_one<C>(f0, fad, stage(0), 0, r);
        }

        // Slice t in stage t%4, fragments of its first k-step already in f0:
        //   step 0: MFMAs on f0, reads of step 1 into f1, first half of the
        //           direct loads of slice t+3 into stage (t+3)%4 (that stage was
        //           last read in slice t-1, before the previous barrier);
        //   wait until this wave's loads of slice t+1 have landed, barrier
        //           (everyone's have, and everyone's reads of slice t are done);
        //   step 1: MFMAs on f1, reads of step 0 of slice t+1 into f0, second
        //           half of the direct loads of slice t+3.
        // Loads issued after slice t+1's when waiting: all D of slice t+2 and
        // the first D/2 of slice t+3, hence vmcnt(3D/2) in the steady state.
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
                dma.template issue_one<FULL, decltype(d)::value + D / 2>(kt, kt & 3);
            };
            kstep<C, T, true, ISSUE>(f0, f1, acc, fad, st, 1, dma_lo);
            if constexpr (NEXT) {
                wait_vmcnt<decltype(wait)::value>();
                // with nothing left in flight, slice t + 1 is the last one
                if constexpr (GEN && decltype(wait)::value == 0)
                    fix_last_slice<C, T>(args, m0, n0, t + 1, stage((t + 1) & 3));
                __syncthreads();
            }
            kstep<C, T, NEXT, ISSUE>(f1, f0, acc, fad, stage((t + 1) & 3), 0, dma_hi);
        };
        using yes = std::true_type;
        using no = std::false_type;
        using none = std::integral_constant<int, 0>;
        using full = std::integral_constant<int, 1>;
        using last = std::integral_constant<int, 2>;
        using w_steady = std::integral_constant<int, 3 * D / 2>;
        using w_two = std::integral_constant<int, D>;
        using w0 = std::integral_constant<int, 0>;
        int t = 0;
        for (; t + 4 < nk; ++t)
            slice(t, full{}, w_steady{}, yes{});
        if (t + 3 < nk) {
            slice(t, last{}, w_steady{}, yes{});
            ++t;
        }
        if (t + 3 == nk && t < nk) {
            slice(t, none{}, w_two{}, yes{});
            ++t;
        }
        if (t + 2 == nk && t < nk) {
            slice(t, none{}, w0{}, yes{});
            ++t;
        }
        if (t + 1 == nk)
            slice(t, none{}, w0{}, no{});

        store_tile_wave<C, T, EPI, !GEN>(args, acc, m0, n0, wm, wn, wave, lane, lds0, nk);
        // every wave is done reading LDS before the next tile's loads land
        __syncthreads();
    }
}

template <class C, class T, int EPI>
hipError_t launch_typed(const GemmArgs &a, bool gen, int grid, hipStream_t stream) {
    if (gen)
        hipLaunchKernelGGL((gemm_tiled_kernel<C, T, EPI, true>), dim3(grid), dim3(NTHREADS), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_tiled_kernel<C, T, EPI, false>), dim3(grid), dim3(NTHREADS), 0, stream, a);
    return hipGetLastError();
}

template <class C, class T>
hipError_t launch_epi(int epi, const GemmArgs &a, bool gen, int grid, hipStream_t stream) {
    switch (epi) {
    case EPI_NONE: return launch_typed<C, T, EPI_NONE>(a, gen, grid, stream);
    case EPI_BIAS: return launch_typed<C, T, EPI_BIAS>(a, gen, grid, stream);
    default: return launch_typed<C, T, EPI_BIAS_GELU_TANH>(a, gen, grid, stream);
    }
}

template <class C>
hipError_t launch_cfg(int dtype, int epi, const GemmArgs &a, bool aligned, int num_cu, hipStream_t stream) {
    const int tiles = ((a.M + C::BM - 1) / C::BM) * ((a.N + C::BN - 1) / C::BN);
    int grid = tiles;
    const int slots = num_cu * C::OCCUPANCY;
    if (num_cu > 0 && tiles > slots) {
        // OCCUPANCY workgroups per CU, rounded down to a multiple of the XCD count
        grid = slots >= tile::NUM_XCD ? slots - slots % tile::NUM_XCD : slots;
    }
    return dtype == 0 ? launch_epi<C, F16>(epi, a, !aligned, grid, stream)
                      : launch_epi<C, BF16>(epi, a, !aligned, grid, stream);
}

}  // namespace

int tiled_occupancy(int tiles) {
    switch (tiles) {
    case TILES_256x128: return Cfg<256, 128>::OCCUPANCY;
    case TILES_128x256: return Cfg<128, 256>::OCCUPANCY;
    case TILES_128x128: return Cfg<128, 128>::OCCUPANCY;
    default: return Cfg<256, 256>::OCCUPANCY;
    }
}

hipError_t launch_tiled_vec(int dtype, int epi, const GemmArgs &a, bool aligned, int tiles, int num_cu,
                            hipStream_t stream) {
    switch (tiles) {
    case TILES_256x128: return launch_cfg<Cfg<256, 128>>(dtype, epi, a, aligned, num_cu, stream);
    case TILES_128x256: return launch_cfg<Cfg<128, 256>>(dtype, epi, a, aligned, num_cu, stream);
    case TILES_128x128: return launch_cfg<Cfg<128, 128>>(dtype, epi, a, aligned, num_cu, stream);
    default: return launch_cfg<Cfg<256, 256>>(dtype, epi, a, aligned, num_cu, stream);
    }
}

}  // namespace tg
