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
//   * tile BM x BN with BM, BN in {128, 256}, k-slices of BK in {32, 64}, a
//     ring of S LDS stages and 4 or 8 wave64s in a WGM x WGN grid, each wave
//     owning a BM/WGM x BN/WGN block of C as v_mfma_f32_32x32x16
//     accumulators in AGPRs (256 fp32 values per lane at 256 x 256 on 4
//     waves); the configuration is a template parameter and the host picks
//     one per shape (the default: 256 x 256, BK = 32, 4 stages, 4 waves);
//   * the stages (4 x 32 KB of the 160 KB LDS at 256 x 256, BK = 32) are
//     filled by buffer loads that write LDS directly (buffer_load_dwordx4 ...
//     lds): no staging registers, no LDS store instructions; with S >= 3
//     stages each slice is requested S - 2 slices before it is used, with 2
//     stages right after the barrier that frees its stage; one barrier per
//     slice, before its last k-step;
//   * LDS holds the A tiles of all stages, then their B tiles, and the k-loop
//     is unrolled over the ring, so a fragment read names its stage in the
//     instruction's offset field instead of adding it to the lane's address
//     (24 fewer vector adds per slice at 256 x 256; the per-lane address
//     registers hold the offsets within a tile, plus the B region's start);
//   * A is staged as [BM m][BK k] (k-contiguous, what a 16-bit MFMA operand
//     holds per lane) and read with ds_read_b128; B stays [BK k][BN n] as in
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
//     consecutive output columns of a row; the accumulators of a tile start
//     at the bias of their columns, so after the k-loop only GELU(tanh) and
//     the rounding are left, and each wave's block of C then goes through
//     LDS 32 rows at a time and leaves as row segments;
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

using namespace direct;
constexpr uint32_t OOB_BUMP = 0x80000000u;        // + offset < 2^31 - 64 KiB -> beyond the operand's buffer
constexpr int LDS_BYTES = 160 * 1024;             // per CU on gfx950

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Everything that follows from the configuration: tile BM x BN, k-slice BK,
// S LDS stages, WGM x WGN waves.  Each wave owns WM x WN = (BM/WGM) x
// (BN/WGN) of C as I x J accumulators of 32 x 32, and takes KS = BK/16
// k-steps per slice.  Per k-slice and wave: QA direct loads of A (RPD rows
// of 2 BK bytes each) and QB of B (1 KB = RB k-rows each).
template <int BM_, int BN_, int BK_ = 32, int S_ = 4, int WGM_ = 2, int WGN_ = 2>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_, WGM = WGM_, WGN = WGN_;
    static_assert((BM == 128 || BM == 256) && (BN == 128 || BN == 256), "tile sizes");
    static_assert(BK == 32 || BK == 64, "k-slice");
    static constexpr int WAVES = WGM * WGN;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int I = WM / 32, J = WN / 32;
    static_assert(I >= 1 && J >= 1, "at least one 32 x 32 block per wave");
    static constexpr int KS = BK / 16;                      // k-steps per slice
    static constexpr int ACH = BK / 8;                      // 16-byte chunks per A row of the stage
    static constexpr int A_ROW = 2 * BK;                    // bytes per row of the A stage
    static constexpr int A_BYTES = BM * BK * 2;             // [BM m][BK k]
    static constexpr int B_BYTES = BK * BN * 2;             // [BK k][BN n]
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int B_ROW = 2 * BN;                    // bytes per k-row of the B stage
    static constexpr int CPR = BN / 8;                      // 16-byte chunks per B row
    static constexpr int RPD = 1024 / A_ROW;                // A rows per direct load
    static constexpr int RB = 1024 / B_ROW;                 // B k-rows per direct load
    static constexpr int A_ROWS_PER_WAVE = BM / WAVES;
    static constexpr int B_ROWS_PER_WAVE = BK / WAVES;
    static constexpr int QA = A_ROWS_PER_WAVE / RPD, QB = B_ROWS_PER_WAVE / RB;
    static_assert(QA * RPD == A_ROWS_PER_WAVE && QB * RB == B_ROWS_PER_WAVE && QA >= 1 && QB >= 1, "load split");
    static constexpr int D = QA + QB;                       // direct loads per slice per wave
    static constexpr int READS = I + 2 * J;                 // fragment reads per k-step
    static constexpr int MFMAS = I * J;                     // MFMAs per k-step
    static_assert(S >= 2 && S * STAGE_BYTES <= LDS_BYTES, "stages fit LDS");
    // with S >= 3 stages each k-step of slice t issues D/KS loads of slice
    // t + S - 1; with 2 stages the last k-step issues all D loads of slice t + 2
    static_assert(S == 2 ? D <= 2 * MFMAS : (D % KS == 0 && D / KS <= MFMAS), "loads fit the k-steps");
    static constexpr int OCCUPANCY = (S * STAGE_BYTES <= LDS_BYTES / 2 && WAVES == 4) ? 2 : 1;   // workgroups per CU
    // LDS: the A tiles of the S stages, then their B tiles
    static constexpr int B_REGION = S * A_BYTES;
    // this wave's loads pending, when waiting for slice t + 1 at the barrier of
    // slice t in the steady state: slices t + 2 .. t + S - 2 and the part of
    // slice t + S - 1 issued before the barrier
    static constexpr int WAIT_STEADY = S == 2 ? 0 : (S - 3) * D + (KS - 1) * (D / KS);
};

// A row = BK k = ACH chunks of 16 B.  A fragment read takes one logical
// chunk from 32 consecutive rows.  ACH = 4 (64-byte rows): any 8 consecutive
// rows of one parity and any 16 consecutive rows of one residue mod 4 use 4
// different slots; ACH = 8 (128-byte rows, two per 256-byte bank cycle): any
// 8 consecutive rows (aligned to 8) use 8 different slots and any 16
// consecutive rows (aligned to 16) 16 different (row parity, slot) pairs.
// Both keep 32-bank (8 lanes x 16 B) and 64-bank (16 lanes) passes conflict
// free.
template <int ACH>
__device__ __forceinline__ int a_swz(int row) {
    if constexpr (ACH == 4)
        return ((row >> 1) ^ (row >> 2)) & 3;
    else
        return (row & 7) ^ ((row >> 3) & 1);
}

// B row = BN n = 32 or 16 chunks.  A transposed read pass touches 4
// consecutive k-rows (k % 4 = 0..3) and 2 (32-bank pass) or 4 (64-bank pass)
// adjacent chunks; g(k%4) = {0, 10, 4, 14} gives those 4 rows distinct bits
// 1-2 and distinct bits 2-3 of the slot, so every pass hits distinct banks
// (the 64 banks span 256 bytes, so only the chunk index mod 16 matters).
__device__ __forceinline__ int b_swz(int k) { return ((k & 1) ? 10 : 0) ^ ((k & 2) ? 4 : 0); }

// LDS addresses of one stage's A and B tiles.  All stages' A tiles come
// first and then all B tiles, so that with the stage known at compile time
// (the k-loop is unrolled over the ring) a fragment read's address is the
// lane's register plus an instruction offset below 64 KiB, with no add per
// read, wherever the A tiles and the B tiles each span at most 64 KiB.
struct StageAt {
    uint32_t a, b;
};
template <class C>
__device__ __forceinline__ StageAt stage_at(uint32_t lds0, int st) {
    return StageAt{lds0 + (uint32_t)st * (uint32_t)C::A_BYTES,
                   lds0 + (uint32_t)C::B_REGION + (uint32_t)st * (uint32_t)C::B_BYTES};
}

// Per-lane addressing of the D direct loads that fill one stage.  Wave w,
// lane L:
//   A load q < QA: tile rows A_ROWS_PER_WAVE w + RPD q + L/ACH, physical
//      chunk L%ACH -> logical chunk c = L%ACH ^ a_swz(row) (8 k);
//      destination the stage's A tile + A_BYTES/WAVES w + 1024 q;
//   B load q < QB: k-row B_ROWS_PER_WAVE w + RB q + L/CPR, physical chunk
//      L%CPR -> logical chunk c = L%CPR ^ b_swz(k) (8 n); destination
//      the stage's B tile + B_BYTES/WAVES w + 1024 q.
// Loads of one operand share m0 in groups of four (their destination is m0
// + 4096 (q/4), the group's m0, plus the instruction offset 1024 (q%4),
// which is also added to the memory offset; the lane offsets subtract it
// back).  So that they stay non-negative, the buffers start 4 KB before the
// operands (offsets are operand offsets + 4096) and are 4 KB longer.
// Lanes whose rows lie at m >= M (A) or whose whole chunk lies at n >= N (B)
// only feed outputs that are never stored: their offset is 2^31, beyond every
// buffer, so they read zeros.  The slices of the steady loop (all but the
// prologue's and the last) lie inside [0, K - 1), so there every other A
// lane's chunk is inside A, and the slice's k offset goes into the load's
// soffset, with no vector add.  B does the same when SOFF_B: with N % 8 == 0
// (so N >= 8) a B chunk that crosses N ends inside the next k-row, which
// exists; with N < 8 it could run past B's last row, so the other instance
// adds the k offset to the lane offset, where the range check sees it.  The
// prologue's and the last slice add it to the lane offset too and send
// k >= K beyond the buffer, as the range check zeroes them.
template <class C, bool SOFF_B>
struct Dma {
    static constexpr uint32_t SHIFT = 4096;
    i32x4 ra, rb;
    uint32_t a_off[C::QA];   // buffer offset of this lane's A chunk for load q, k0 = 0, minus 1024 (q%4); 2^31 for m >= M
    int a_k[C::QA];          // first k of the lane's A chunk of load q within the slice
    uint32_t b_off[C::QB];   // the same for B; 2^31 for a chunk at n >= N
    int b_k[C::QB];          // k-row of load q within the slice
    uint32_t b_row;          // bytes per row of B
    uint32_t m0_a, m0_b;     // LDS destinations of load q = 0 in stage 0
    int K;

    __device__ __forceinline__ Dma(const GemmArgs &g, int m0, int n0, int wave, int lane, uint32_t lds0) {
        ra = rsrc_words((const char *)g.A - SHIFT, 2u * (uint32_t)g.M * (uint32_t)g.K + SHIFT);
        rb = rsrc_words((const char *)g.B - SHIFT, 2u * (uint32_t)g.K * (uint32_t)g.N + SHIFT);
        K = g.K;
        const int arow = C::A_ROWS_PER_WAVE * wave + (int)((unsigned)lane / C::ACH);
        b_row = 2u * (uint32_t)g.N;
#pragma unroll
        for (int q = 0; q < C::QA; ++q) {
            const int row = arow + C::RPD * q;   // row within the tile
            a_k[q] = 8 * ((int)((unsigned)lane % C::ACH) ^ a_swz<C::ACH>(row));
            a_off[q] = m0 + row < g.M ? SHIFT - 1024u * (q & 3) +
                                            2u * ((uint32_t)(m0 + row) * (uint32_t)g.K + (uint32_t)a_k[q])
                                      : OOB_BUMP;
        }
#pragma unroll
        for (int q = 0; q < C::QB; ++q) {
            const int k = C::B_ROWS_PER_WAVE * wave + C::RB * q + (int)((unsigned)lane / C::CPR);
            const int c = (int)((unsigned)lane % C::CPR) ^ b_swz(k);
            b_k[q] = k;
            b_off[q] = n0 + 8 * c < g.N ? SHIFT - 1024u * (q & 3) + (uint32_t)k * b_row + 2u * (uint32_t)(n0 + 8 * c)
                                        : OOB_BUMP;
        }
        m0_a = lds0 + (uint32_t)(C::A_BYTES / C::WAVES) * (uint32_t)wave;
        m0_b = lds0 + (uint32_t)C::B_REGION + (uint32_t)(C::B_BYTES / C::WAVES) * (uint32_t)wave;
    }

    // Direct load d (0..D-1) of k-slice kt into LDS stage st: A load d for
    // d < QA, B load d - QA otherwise.  FULL: the slice lies inside [0, K), so
    // no lane needs the K mask (only the last slice can be partial).
    template <bool FULL, int DI>
    __device__ __forceinline__ void issue_one(int kt, int st) const {
        const int k0 = __builtin_amdgcn_readfirstlane(kt * C::BK);   // uniform: address arithmetic in SGPRs
        if constexpr (DI < C::QA) {
            constexpr int q = DI;
            const uint32_t m0 = m0_a + (uint32_t)st * (uint32_t)C::A_BYTES + 4096u * (q >> 2);
            if constexpr (FULL) {
                dma16s<1024 * (q & 3)>(ra, a_off[q], 2u * (uint32_t)k0, m0);
            } else {
                const uint32_t off = (a_off[q] + 2u * (uint32_t)k0) | ((k0 + a_k[q] < K) ? 0u : OOB_BUMP);
                dma16<1024 * (q & 3)>(ra, off, m0);
            }
        } else {
            constexpr int q = DI - C::QA;
            const uint32_t m0 = m0_b + (uint32_t)st * (uint32_t)C::B_BYTES + 4096u * (q >> 2);
            if constexpr (FULL && SOFF_B) {
                dma16s<1024 * (q & 3)>(rb, b_off[q], __builtin_amdgcn_readfirstlane((uint32_t)k0 * b_row), m0);
            } else if constexpr (FULL) {
                dma16<1024 * (q & 3)>(rb, b_off[q] + (uint32_t)k0 * b_row, m0);
            } else {
                const uint32_t off = (b_off[q] + (uint32_t)k0 * b_row) | ((k0 + b_k[q] < K) ? 0u : OOB_BUMP);
                dma16<1024 * (q & 3)>(rb, off, m0);
            }
        }
    }

    template <int... DI>
    __device__ __forceinline__ void issue_seq(int kt, int st, std::integer_sequence<int, DI...>) const {
        (issue_one<false, DI>(kt, st), ...);
    }

    // Request k-slice kt into LDS stage st (prologue: no slice is partial
    // there unless it is also the last, which the K mask then covers).
    __device__ __forceinline__ void issue(int kt, int st) const {
        issue_seq(kt, st, std::make_integer_sequence<int, C::D>{});
    }
};

// Per-lane LDS byte offsets of the fragment reads of k-step s (16 k each),
// for A from the stage's A tile, for B from the start of all stages' B tiles
// (the stage's place among them is added to it):
//   A, ds_read_b128: row wm*WM + 32 i + l%32, logical chunk 2 s + l/32;
//   B, ds_read_b64_tr_b16 twice (k 0..3 and 4..7 of the lane's 8): lane
//      16 G + q addresses k-row 16 s + 8 (G/2) + q/4 (+4), columns
//      wn*WN + 32 j + 16 (G%2) + 4 (q%4) .. +3, so that lane l receives
//      column wn*WN + 32 j + l%32, k = 16 s + 8 (l/32) + 0..7.
template <class C>
struct FragAddr {
    uint32_t a[C::KS][C::I];   // [s][i]
    uint32_t b[C::J];          // step 0, first read; step s is + 16 s rows, the second read + 4 rows

    __device__ __forceinline__ FragAddr(int wm, int wn, int lane) {
        const int lr = lane & 31;
#pragma unroll
        for (int i = 0; i < C::I; ++i) {
            const int row = wm * C::WM + 32 * i + lr;
            const int sw = a_swz<C::ACH>(row);
#pragma unroll
            for (int s = 0; s < C::KS; ++s) {
                const int c = 2 * s + (lane >> 5);
                a[s][i] = (uint32_t)(C::A_ROW * row) + 16u * (uint32_t)(c ^ sw);
            }
        }
        const int G = lane >> 4;
        const int q = lane & 15;
        const int kr = 8 * (G >> 1) + (q >> 2);      // k-row for s = 0, first read; kr % 4 = q / 4
        const int bsw = b_swz(kr);
#pragma unroll
        for (int j = 0; j < C::J; ++j) {
            const int n = wn * C::WN + 32 * j + 16 * (G & 1) + 4 * (q & 3);
            const int c = (n >> 3) ^ bsw;
            b[j] = (uint32_t)C::B_REGION + (uint32_t)C::B_ROW * (uint32_t)kr + 16u * (uint32_t)c +
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
__device__ __forceinline__ void read_one(Frag<C> &f, const FragAddr<C> &ad, StageAt stage, int s, int r) {
    if (r < C::I) {
        f.a[r] = lds_u4(stage.a + ad.a[s][r]);
    } else {
        const int j = (r - C::I) >> 1;
        // ad.b holds the B region's base, so that what is added to it is the
        // stage's place within the region (an instruction offset)
        const uint32_t b = (stage.b - (uint32_t)C::B_REGION) + ad.b[j] + (uint32_t)(16 * C::B_ROW * s);
        if (((r - C::I) & 1) == 0) {
            const u32x2 v = lds_tr(b);
            f.b[j].x = v.x;
            f.b[j].y = v.y;
        } else {
            const u32x2 v = lds_tr(b + 4u * (uint32_t)C::B_ROW);
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

// A k-step with H direct loads: load p (0..H-1) goes after MFMA
// (p*M/H + 1) mod M (M MFMAs per k-step).
template <class C, int Q, int H>
struct DmaAfter {
    static constexpr int pos(int p) { return ((p * C::MFMAS) / H + 1) % C::MFMAS; }
    static constexpr int find(int p) { return p >= H ? -1 : (pos(p) == Q ? p : find(p + 1)); }
    static constexpr int P = H > 0 ? find(0) : -1;
};

template <class C, int R0, int... R>
__device__ __forceinline__ void read_range(Frag<C> &nxt, const FragAddr<C> &ad, StageAt rstage, int rs,
                                           std::integer_sequence<int, R...>) {
    (read_one<C>(nxt, ad, rstage, rs, R0 + R), ...);
}

// One k-step in a fixed issue order: MFMA Q (A block Q/J x B block Q%J),
// then the fragment reads of the next step that follow it, then the direct
// loads placed after it (`dma(p)`, p = 0..H-1; with H > M some MFMAs are
// followed by two).  sched_barrier keeps the compiler from regrouping:
// spreading the direct loads lets the memory pipeline take them while the
// matrix unit stays busy.
template <class C, class T, bool READ, int H, int Q, typename DmaFn>
__device__ __forceinline__ void kstep_one(const Frag<C> &cur, Frag<C> &nxt, f32x16 (&acc)[C::I][C::J],
                                          const FragAddr<C> &ad, StageAt rstage, int rs, DmaFn &dma) {
    acc[Q / C::J][Q % C::J] = T::mfma32(cur.b[Q % C::J], cur.a[Q / C::J], acc[Q / C::J][Q % C::J]);
    if constexpr (READ) {
        constexpr int LO = ReadsAfter<C, Q>::LO, HI = ReadsAfter<C, Q>::HI;
        if constexpr (HI > LO)
            read_range<C, LO>(nxt, ad, rstage, rs, std::make_integer_sequence<int, HI - LO>{});
    }
    if constexpr (H <= C::MFMAS) {
        if constexpr (DmaAfter<C, Q, H>::P >= 0)
            dma(std::integral_constant<int, DmaAfter<C, Q, H>::P>{});
    } else {   // two per MFMA for the first H - M MFMAs
        constexpr int P0 = Q < H - C::MFMAS ? 2 * Q : (H - C::MFMAS) + Q;
        dma(std::integral_constant<int, P0>{});
        if constexpr (Q < H - C::MFMAS)
            dma(std::integral_constant<int, P0 + 1>{});
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <class C, class T, bool READ, int H, typename DmaFn, int... Q>
__device__ __forceinline__ void kstep_seq(const Frag<C> &cur, Frag<C> &nxt, f32x16 (&acc)[C::I][C::J],
                                          const FragAddr<C> &ad, StageAt rstage, int rs, DmaFn &dma,
                                          std::integer_sequence<int, Q...>) {
    (kstep_one<C, T, READ, H, Q>(cur, nxt, acc, ad, rstage, rs, dma), ...);
}

// One k-step: MFMAs on `cur`; with READ the fragments of k-step rs of the
// stage at rstage are read into `nxt`; H direct loads through dma(p).
template <class C, class T, bool READ, int H, typename DmaFn>
__device__ __forceinline__ void kstep(const Frag<C> &cur, Frag<C> &nxt, f32x16 (&acc)[C::I][C::J],
                                      const FragAddr<C> &ad, StageAt rstage, int rs, DmaFn dma) {
    kstep_seq<C, T, READ, H>(cur, nxt, acc, ad, rstage, rs, dma, std::make_integer_sequence<int, C::MFMAS>{});
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
__device__ __forceinline__ void fix_last_slice(const GemmArgs &g, int m0, int n0, int kl, StageAt stage) {
    const int k0 = kl * C::BK;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    if (g.K % 8 != 0 && lane < C::A_ROWS_PER_WAVE) {
        const __amdgpu_buffer_rsrc_t ra = tile::buffer_of(g.A, 2u * (uint32_t)g.M * (uint32_t)g.K);
        const int r = C::A_ROWS_PER_WAVE * wave + lane;   // tile row r was loaded by this wave
        const int cp = (g.K - k0) >> 3;          // the crossing chunk (< ACH: the slice holds K - 1)
        const int v = (g.K - k0) & 7;            // its elements below K
        const uint32_t row = (uint32_t)(m0 + r); // rows >= M read zero (beyond the buffer)
        const uint32_t base = 2u * (row * (uint32_t)g.K + (uint32_t)(k0 + 8 * cp));
        uint16_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            e[q] = q < v ? __builtin_amdgcn_raw_buffer_load_b16(ra, (int)(base + 2u * q), 0, 0) : (uint16_t)0;
        const u32x4 chunk = {pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7])};
        *(__attribute__((address_space(3))) u32x4 *)(uintptr_t)(stage.a + (uint32_t)(C::A_ROW * r) +
                                                                16u * (uint32_t)(cp ^ a_swz<C::ACH>(r))) = chunk;
    }
    if (g.N % 8 != 0 && n0 <= g.N - 1 && g.N - 1 < n0 + C::BN) {
        const int r = g.K - 1 - k0;              // B's last row, loaded by wave r / B_ROWS_PER_WAVE
        if (tid == 64 * (r / C::B_ROWS_PER_WAVE)) {
            const __amdgpu_buffer_rsrc_t rb = tile::buffer_of(g.B, 2u * (uint32_t)g.K * (uint32_t)g.N);
            const int c = (g.N - 1 - n0) >> 3;
            const uint32_t base = 2u * ((uint32_t)(g.K - 1) * (uint32_t)g.N + (uint32_t)(n0 + 8 * c));
            uint16_t e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                e[q] = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)(base + 2u * q), 0, 0);
            const u32x4 chunk = {pack2(e[0], e[1]), pack2(e[2], e[3]), pack2(e[4], e[5]), pack2(e[6], e[7])};
            *(__attribute__((address_space(3))) u32x4 *)(uintptr_t)(stage.b + (uint32_t)C::B_ROW * r +
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
    static constexpr int PER_A = C::A_BYTES / BUF;             // buffers in a stage's A tile
    static constexpr int PER_STAGE = PER_A + C::B_BYTES / BUF; // and in its B tile
    static_assert(PER_A * BUF == C::A_BYTES && (PER_STAGE - PER_A) * BUF == C::B_BYTES, "buffers tile the stage");
    static_assert(PER_STAGE >= 1 && (C::WAVES + PER_STAGE - 1) / PER_STAGE <= C::S - 1,
                  "wave buffers fit the stages other than the last slice's");
    static __device__ __forceinline__ uint32_t swz(int row) {
        return (uint32_t)((row ^ (row / CPRW)) & (CPRW - 1));
    }
    // wave w's buffer: in the stages after the last slice's (nk - 1) % S
    static __device__ __forceinline__ uint32_t buffer(uint32_t lds0, int nk, int w) {
        const StageAt st = stage_at<C>(lds0, (nk + w / PER_STAGE) % C::S);
        const int p = w % PER_STAGE;
        return p < PER_A ? st.a + (uint32_t)(p * BUF) : st.b + (uint32_t)((p - PER_A) * BUF);
    }
};

// The accumulators of a tile start at the bias of their columns (zero
// without a bias): the fused epilogue's bias then enters the fp32 sum first
// instead of last, which is another rounding order of the same sum (integer
// valued sums stay exact), and the epilogue after the k-loop is left with
// GELU and the conversion.  Element 4 q + r of block (i, j) of lane l holds
// column wn WN + 32 j + 8 q + 4 (l / 32) + r for every i.  Range-checked
// loads: columns past N read zero.
template <class C, class T, int EPI, bool ALIGNED>
__device__ __forceinline__ void init_acc(f32x16 (&acc)[C::I][C::J], const GemmArgs &args, int n0, int wn,
                                         int lane) {
    f32x16 first[C::J];
#pragma unroll
    for (int j = 0; j < C::J; ++j)
        first[j] = f32x16{};
    if constexpr (EPI != EPI_NONE) {
        const __amdgpu_buffer_rsrc_t rb = tile::buffer_of(args.bias, 2u * (uint32_t)args.N);
        const int lh = lane >> 5;
#pragma unroll
        for (int j = 0; j < C::J; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t off = 2u * (uint32_t)(n0 + wn * C::WN + 32 * j + 8 * q + 4 * lh);
                uint16_t e[4];
                if constexpr (ALIGNED) {   // N % 8 == 0: a group is all inside or all outside
                    const u32x2 raw = __builtin_amdgcn_raw_buffer_load_b64(rb, (int)off, 0, 0);
                    e[0] = (uint16_t)(raw.x & 0xffff);
                    e[1] = (uint16_t)(raw.x >> 16);
                    e[2] = (uint16_t)(raw.y & 0xffff);
                    e[3] = (uint16_t)(raw.y >> 16);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        e[r] = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)(off + 2u * r), 0, 0);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    first[j][4 * q + r] = T::to_f32(e[r]);
            }
    }
#pragma unroll
    for (int i = 0; i < C::I; ++i)
#pragma unroll
        for (int j = 0; j < C::J; ++j)
            acc[i][j] = first[j];
}

// C leaves with the non-temporal cache policy: nothing reads it again in the
// kernel, and lines of C kept in L2 would only displace the A and B panels
// the other tiles of the XCD still read (≈1 % on every tiled shape measured).
constexpr int kStoreCpol = 2;

template <class C, class T, int EPI, bool ALIGNED>
__device__ __forceinline__ void store_tile_wave(const GemmArgs &args, const f32x16 (&acc)[C::I][C::J], int m0,
                                                int n0, int wm, int wn, int wave, int lane, uint32_t lds0,
                                                int nk) {
    using W = WaveStage<C>;
    const int M = args.M, N = args.N;
    const int lr = lane & 31;
    const int lh = lane >> 5;
    // the stage of the last slice is (nk - 1) % S; the next ones are free
    const uint32_t buf = W::buffer(lds0, nk, wave);
    const __amdgpu_buffer_rsrc_t rc = tile::buffer_of(args.C, 2u * (uint32_t)M * (uint32_t)N);
#pragma unroll
    for (int i = 0; i < C::I; ++i) {
#pragma unroll
        for (int j = 0; j < C::J; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint16_t o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)   // the bias is in the accumulator already
                    o[r] = T::from_f32(EPI == EPI_BIAS_GELU_TANH ? gelu_tanh(acc[i][j][4 * q + r])
                                                                 : acc[i][j][4 * q + r]);
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
                __builtin_amdgcn_raw_buffer_store_b128(v, rc, (int)off, 0, kStoreCpol);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t off = (m < M && n + e < N) ? base + 2u * e : tile::OOB;
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(v[e >> 1] >> (16 * (e & 1))), rc, (int)off, 0,
                                                          kStoreCpol);
                }
            }
        }
    }
}

// f(integral_constant<int, I>) for I = 0 .. N-1, in order.
template <typename F, int... I>
__device__ __forceinline__ void for_each_index(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}

// Prologue wait for slice 0 when `issued` slices (1..P) were requested:
// (issued - 1) D loads of this wave are younger than slice 0's.
template <int D, int P>
__device__ __forceinline__ void wait_prologue(int issued) {
    if constexpr (P <= 1) {
        wait_vmcnt<0>();
    } else {
        if (issued >= P)
            wait_vmcnt<(P - 1) * D>();
        else
            wait_prologue<D, P - 1>(issued);
    }
}

// Persistent: the grid has at most OCCUPANCY workgroups per CU, and
// workgroup g computes tiles g, g + G, g + 2G, ... (G = grid size, a
// multiple of the 8 XCDs when the tile count allows, so every tile of a
// workgroup stays on its XCD in the raster), which removes the dispatch gap
// between tiles.
template <class C, class T, int EPI, bool GEN>
__global__ __launch_bounds__(C::THREADS, C::OCCUPANCY) void gemm_tiled_kernel(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) u32x4 smem[C::S * C::STAGE_BYTES / 16];
    constexpr int D = C::D, S = C::S, KS = C::KS;
    // slice t requests slice t + LEAD: S - 1 with S >= 3 stages (before and
    // after its barrier), 2 with two stages (after its barrier)
    constexpr int LEAD = S == 2 ? 2 : S - 1;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / C::WGN;
    const int wn = wave % C::WGN;
    const uint32_t lds0 = lds_address(smem);
    auto stage = [&](int st) { return stage_at<C>(lds0, st); };
    const int tiles_m = (args.M + C::BM - 1) / C::BM;
    const int tiles_n = (args.N + C::BN - 1) / C::BN;
    const int total = tiles_m * tiles_n;
    const int nk = (args.K + C::BK - 1) / C::BK;

    for (int w = blockIdx.x; w < total; w += gridDim.x) {
        // The lane id is made opaque per tile so that the per-lane addresses
        // below are recomputed for each tile instead of being hoisted out of
        // the tile loop, where they would stay live through the k-loop.
        int lane = threadIdx.x & 63;
        asm volatile("" : "+v"(lane));
        const FragAddr<C> fad(wm, wn, lane);
        int tm, tn;
        tile::tile_of_index(tiles_m, tiles_n, w, args.group_m, tm, tn);
        const int m0 = tm * C::BM;
        const int n0 = tn * C::BN;
        const Dma<C, !GEN> dma(args, m0, n0, wave, lane, lds0);

        f32x16 acc[C::I][C::J];
        init_acc<C, T, EPI, !GEN>(acc, args, n0, wn, lane);

        Frag<C> f[2];
        // Prologue: request slices 0 .. min(LEAD, nk) - 1, wait for slice 0.
        // The previous tile's C stores only add to the count: loads complete
        // in order, so slice 0 has landed once no more than the younger
        // loads are pending.
        if (nk > 0) {
#pragma unroll
            for (int p = 0; p < LEAD; ++p)
                if (p < nk)
                    dma.issue(p, p);
            const int issued = nk < LEAD ? nk : LEAD;
            wait_prologue<D, LEAD>(issued);
            if constexpr (GEN)
                if (nk == 1)
                    fix_last_slice<C, T>(args, m0, n0, 0, stage(0));
        }
        __syncthreads();
        if (nk > 0) {
#pragma unroll
            for (int r = 0; r < C::READS; ++r)
                read_one<C>(f[0], fad, stage(0), 0, r);
        }

        // Slice t in stage t % S, fragments of its first k-step already in f[0]:
        //   k-steps 0 .. KS-2: MFMAs on f[s % 2], reads of step s + 1 into
        //       f[(s + 1) % 2] and (S >= 3) D/KS direct loads each of slice
        //       t + S - 1 into stage (t - 1) % S, last read in slice t - 1,
        //       before its barrier;
        //   wait until this wave's loads of slice t + 1 have landed, barrier
        //       (everyone's have, and everyone's reads of slice t are done);
        //   k-step KS-1: MFMAs, reads of step 0 of slice t + 1 into f[0], and
        //       the last D/KS loads of slice t + S - 1 (S >= 3) or all D loads
        //       of slice t + 2 into stage t % 2, just freed (S == 2).
        // RES: t % S when known at compile time (the stages' LDS addresses
        // are then constants), -1 otherwise.  ISSUE: 0 = no loads, 1 = loads
        // of a full slice, 2 = loads of the (possibly partial) last slice.
        // WAIT: this wave's loads younger than slice t + 1's at the barrier.
        // FIX: slice t + 1 is the last one of a GEN shape.
        auto slice = [&](int t, auto res, auto issue, auto wait, auto next, auto fix) __attribute__((always_inline)) {
            constexpr int R = decltype(res)::value;
            constexpr int IK = decltype(issue)::value;
            constexpr bool FULL = IK == 1;
            constexpr bool NEXT = decltype(next)::value;
            constexpr int HP = (S >= 3 && IK != 0) ? D / KS : 0;            // loads per step before the barrier
            constexpr int HL = IK == 0 ? 0 : (S >= 3 ? D / KS : D);         // loads in the last step
            constexpr int BL = S >= 3 ? (KS - 1) * (D / KS) : 0;            // first load index of the last step
            const int r0 = R >= 0 ? R : t % S;
            const int r1 = R >= 0 ? (R + 1) % S : (t + 1) % S;
            const int kst = R >= 0 ? (R + LEAD) % S : (t + LEAD) % S;
            const StageAt st = stage(r0);
            const int kt = t + LEAD;
            auto pre = [&](auto s) __attribute__((always_inline)) {
                constexpr int SI = decltype(s)::value;
                auto dma_s = [&](auto p) __attribute__((always_inline)) {
                    dma.template issue_one<FULL, SI * HP + decltype(p)::value>(kt, kst);
                };
                kstep<C, T, true, HP>(f[SI & 1], f[(SI + 1) & 1], acc, fad, st, SI + 1, dma_s);
            };
            for_each_index(pre, std::make_integer_sequence<int, KS - 1>{});
            if constexpr (NEXT) {
                wait_vmcnt<decltype(wait)::value>();
                if constexpr (GEN && decltype(fix)::value)
                    fix_last_slice<C, T>(args, m0, n0, t + 1, stage(r1));
                __syncthreads();
            }
            auto dma_l = [&](auto p) __attribute__((always_inline)) {
                dma.template issue_one<FULL, BL + decltype(p)::value>(kt, kst);
            };
            kstep<C, T, NEXT, HL>(f[(KS - 1) & 1], f[0], acc, fad, stage(r1), 0, dma_l);
        };
        using yes = std::true_type;
        using no = std::false_type;
        using full = std::integral_constant<int, 1>;
        using last = std::integral_constant<int, 2>;
        using w_steady = std::integral_constant<int, C::WAIT_STEADY>;
        using any = std::integral_constant<int, -1>;
        int t = 0;
        // full slices S at a time, each with its stage fixed at compile time
        for (; t + S - 1 + LEAD < nk - 1; t += S)
            for_each_index([&](auto r) __attribute__((always_inline)) {
                slice(t + decltype(r)::value, r, full{}, w_steady{}, yes{}, no{});
            }, std::make_integer_sequence<int, S>{});
        for (; t + LEAD < nk - 1; ++t)
            slice(t, any{}, full{}, w_steady{}, yes{}, no{});
        if (t + LEAD == nk - 1) {
            slice(t, any{}, last{}, w_steady{}, yes{}, no{});
            ++t;
        }
        // the last LEAD slices request nothing: slice nk - 1 - j waits for
        // its successor with slices t + 2 .. nk - 1 (j - 1 of them) pending
        auto tail = [&](auto jj) __attribute__((always_inline)) {
            constexpr int J = LEAD - 1 - decltype(jj)::value;
            if (t == nk - 1 - J) {
                if constexpr (J == 0)
                    slice(t, any{}, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, no{}, no{});
                else
                    slice(t, any{}, std::integral_constant<int, 0>{}, std::integral_constant<int, (J - 1) * D>{},
                          yes{}, std::integral_constant<bool, J == 1>{});
                ++t;
            }
        };
        for_each_index(tail, std::make_integer_sequence<int, LEAD>{});

        store_tile_wave<C, T, EPI, !GEN>(args, acc, m0, n0, wm, wn, wave, lane, lds0, nk);
        // every wave is done reading LDS before the next tile's loads land
        __syncthreads();
    }
}

template <class C, class T, int EPI>
hipError_t launch_typed(const GemmArgs &a, bool gen, int grid, hipStream_t stream) {
    if (gen)
        hipLaunchKernelGGL((gemm_tiled_kernel<C, T, EPI, true>), dim3(grid), dim3(C::THREADS), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_tiled_kernel<C, T, EPI, false>), dim3(grid), dim3(C::THREADS), 0, stream, a);
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

// The configurations of TileCfg: tile, k-slice, stages, waves.
template <int TILES>
struct CfgOf;
template <> struct CfgOf<TILES_256x256> { using type = Cfg<256, 256, 32, 4>; };
template <> struct CfgOf<TILES_256x128> { using type = Cfg<256, 128, 32, 4>; };
template <> struct CfgOf<TILES_128x256> { using type = Cfg<128, 256, 32, 4>; };
template <> struct CfgOf<TILES_128x128> { using type = Cfg<128, 128, 32, 4>; };
template <> struct CfgOf<TILES_256x256_K64> { using type = Cfg<256, 256, 64, 2>; };
template <> struct CfgOf<TILES_256x128_K64> { using type = Cfg<256, 128, 64, 3>; };
template <> struct CfgOf<TILES_128x256_K64> { using type = Cfg<128, 256, 64, 3>; };
template <> struct CfgOf<TILES_128x128_K64> { using type = Cfg<128, 128, 64, 2>; };
template <> struct CfgOf<TILES_256x256_W8> { using type = Cfg<256, 256, 32, 4, 2, 4>; };

}  // namespace

int tiled_occupancy(int tiles) {
    switch (tiles) {
    case TILES_256x128: return CfgOf<TILES_256x128>::type::OCCUPANCY;
    case TILES_128x256: return CfgOf<TILES_128x256>::type::OCCUPANCY;
    case TILES_128x128: return CfgOf<TILES_128x128>::type::OCCUPANCY;
    case TILES_256x256_K64: return CfgOf<TILES_256x256_K64>::type::OCCUPANCY;
    case TILES_256x128_K64: return CfgOf<TILES_256x128_K64>::type::OCCUPANCY;
    case TILES_128x256_K64: return CfgOf<TILES_128x256_K64>::type::OCCUPANCY;
    case TILES_128x128_K64: return CfgOf<TILES_128x128_K64>::type::OCCUPANCY;
    case TILES_256x256_W8: return CfgOf<TILES_256x256_W8>::type::OCCUPANCY;
    default: return CfgOf<TILES_256x256>::type::OCCUPANCY;
    }
}

hipError_t launch_tiled_vec(int dtype, int epi, const GemmArgs &a, bool aligned, int tiles, int num_cu,
                            hipStream_t stream) {
    switch (tiles) {
    case TILES_256x128: return launch_cfg<CfgOf<TILES_256x128>::type>(dtype, epi, a, aligned, num_cu, stream);
    case TILES_128x256: return launch_cfg<CfgOf<TILES_128x256>::type>(dtype, epi, a, aligned, num_cu, stream);
    case TILES_128x128: return launch_cfg<CfgOf<TILES_128x128>::type>(dtype, epi, a, aligned, num_cu, stream);
    case TILES_256x256_K64:
        return launch_cfg<CfgOf<TILES_256x256_K64>::type>(dtype, epi, a, aligned, num_cu, stream);
    case TILES_256x128_K64:
        return launch_cfg<CfgOf<TILES_256x128_K64>::type>(dtype, epi, a, aligned, num_cu, stream);
    case TILES_128x256_K64:
        return launch_cfg<CfgOf<TILES_128x256_K64>::type>(dtype, epi, a, aligned, num_cu, stream);
    case TILES_128x128_K64:
        return launch_cfg<CfgOf<TILES_128x128_K64>::type>(dtype, epi, a, aligned, num_cu, stream);
    case TILES_256x256_W8:
        return launch_cfg<CfgOf<TILES_256x256_W8>::type>(dtype, epi, a, aligned, num_cu, stream);
    default: return launch_cfg<CfgOf<TILES_256x256>::type>(dtype, epi, a, aligned, num_cu, stream);
    }
}

}  // namespace tg
