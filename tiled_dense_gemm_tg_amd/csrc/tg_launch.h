// tg_launch.h -- internal interface between the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

// Validated arguments of one GEMM; sizes fit in int32 because every operand
// is at most 4 GiB (2^31 16-bit elements).
struct GemmArgs {
    int M, N, K;
    int group_m;           // tiled raster: tile rows per group (>= 1)
    const uint16_t *A;     // M x K row-major
    const uint16_t *B;     // K x N row-major
    const uint16_t *bias;  // N entries or nullptr
    uint16_t *C;           // M x N row-major
};

// dtype: 0 fp16, 1 bf16; epi: 0 none, 1 bias, 2 bias + GELU(tanh).

// Tile configurations of the direct-load kernel (values as tg_tiles in
// tg_gemm.h): tile BM x BN, k-slice BK, LDS stages, waves.
enum TileCfg {
    TILES_256x256 = 1,       // BK 32, 4 stages, 4 waves
    TILES_256x128 = 2,       // BK 32, 4 stages, 4 waves
    TILES_128x256 = 3,       // BK 32, 4 stages, 4 waves
    TILES_128x128 = 4,       // BK 32, 4 stages, 4 waves, 2 workgroups per CU
    TILES_256x256_K64 = 5,   // BK 64, 2 stages, 4 waves
    TILES_256x128_K64 = 6,   // BK 64, 3 stages, 4 waves
    TILES_128x256_K64 = 7,   // BK 64, 3 stages, 4 waves
    TILES_128x128_K64 = 8,   // BK 64, 2 stages, 4 waves, 2 workgroups per CU
    TILES_256x256_W8 = 9,    // BK 32, 4 stages, 8 waves (2 x 4) of 128 x 64
};
constexpr int TILES_LAST = TILES_256x256_W8;

// BM x BN tiles (TileCfg) with 16-byte direct-to-LDS loads, any K and N and
// 2-byte alignment, as long as 2 (M + 256) K and 2 (K + 64) (N + 256) stay
// below 2^31 - 65536.  aligned: K % 8 == 0, N % 8 == 0, A, B, C 16-byte and
// bias 8-byte aligned, which takes the instance without last-slice fix-ups
// and with 16-byte stores throughout.
// Persistent: at most tiled_occupancy(tiles) workgroups per CU (num_cu <= 0:
// one workgroup per tile).
hipError_t launch_tiled_vec(int dtype, int epi, const GemmArgs &a, bool aligned, int tiles, int num_cu,
                            hipStream_t stream);
// Workgroups of configuration `tiles` that fit on one CU at once.
int tiled_occupancy(int tiles);

// 256 x 256 tiles with element-granular loads and stores: any shape.
hipError_t launch_tiled_generic(int dtype, int epi, const GemmArgs &a, hipStream_t stream);

// Split-K workspace of the M <= 16 kernels.  With splits > 1 the K range of
// each output block (16 rows x 64 columns) is divided over `splits`
// workgroups: each writes its fp32 partial block (1024 values) to part and
// counts itself in that block's counter; the last to arrive adds the
// partials in split order (so the result does not depend on the arrival
// order), applies the epilogue, stores C and resets the counter to zero.
// No workgroup waits for another.
struct SplitWs {
    int splits;          // 1: no workspace (part, count unused)
    float *part;         // [block][split][1024], 16-byte aligned; stream-K: [slot][1024]
    uint32_t *count;     // [block], zero before the launch, zero after it
    int streamk = 0;     // > 0: stream-K over this many workgroups (M <= 16 skinny kernel; splits unused)
};
// Workspace layout of the split modes: the per-block arrival counters
// first, in a region of at least 64 KiB (16384 blocks) so that the partial
// blocks after it start at the same place for every shape up to that many
// blocks, and a partial block of one call never lands on the counters of
// another call through the same workspace; then the partial blocks.
constexpr int64_t kSplitCounterBytes = int64_t(64) << 10;
inline int64_t split_counter_bytes(int64_t blocks) {
    const int64_t c = (blocks * 4 + 255) / 256 * 256;
    return c > kSplitCounterBytes ? c : kSplitCounterBytes;
}
// Bytes of workspace for `blocks` output blocks and `splits` splits.
inline size_t split_ws_bytes(int64_t blocks, int splits) {
    if (splits <= 1 || blocks <= 0)
        return 0;
    return (size_t)split_counter_bytes(blocks) + (size_t)blocks * (size_t)splits * 4096u;
}
inline SplitWs split_ws(void *ws, int64_t blocks, int splits) {
    SplitWs w{splits, nullptr, nullptr};
    if (splits > 1) {
        w.count = static_cast<uint32_t *>(ws);
        w.part = reinterpret_cast<float *>(static_cast<char *>(ws) + split_counter_bytes(blocks));
    }
    return w;
}
// Stream-K over `groups` workgroups: the counters of `blocks` slabs, then
// one partial block per (slab, workgroup) pair, groups + blocks - 1 of them.
inline size_t streamk_ws_bytes(int64_t blocks, int groups) {
    if (blocks <= 0)
        return 0;
    return (size_t)split_counter_bytes(blocks) + (size_t)(groups + blocks - 1) * 4096u;
}
inline SplitWs streamk_ws(void *ws, int64_t blocks, int groups) {
    SplitWs w{1, nullptr, nullptr};
    w.streamk = groups;
    w.count = static_cast<uint32_t *>(ws);
    w.part = reinterpret_cast<float *>(static_cast<char *>(ws) + split_counter_bytes(blocks));
    return w;
}

// M <= 64, K % 8 == 0, N % 4 == 0, aligned operands; ws.splits >= 1 (at most
// ceil(K / 32)), its workspace laid out by split_ws for ceil(N / 64) blocks,
// or (M <= 16) ws.streamk workgroups, 1 .. ceil(N / 64) ceil(K / 32), with
// the workspace of streamk_ws.
hipError_t launch_skinny(int dtype, int epi, const GemmArgs &a, const SplitWs &ws, hipStream_t stream);

// Weight-only 4-bit product: packed weights in the layout of launch_w4_pack,
// scales (K/group x N), group in {32, 64, 128, 256}, K % group == 0; any M
// (16-row blocks), any N, 2-byte alignment.  ws.splits >= 1 divides the
// scale groups; its workspace is laid out by split_ws for
// ceil(N / 64) ceil(M / 16) blocks (block = row block x slabs + slab).
hipError_t launch_w4(int dtype, int epi, const GemmArgs &a, const uint8_t *packed, const uint16_t *scales, int group,
                     const SplitWs &ws, hipStream_t stream);
// q: K x N bytes (values 0..15), K % 32 == 0 -> packed (ceil(N/64) * 32 * K bytes).
hipError_t launch_w4_pack(int K, int N, const uint8_t *q, uint8_t *packed, hipStream_t stream);

// Attention forward, BSHD layout, head dim 128: O = softmax(scale Q K^T) V.
struct AttnArgs {
    int B, Sq, Sk, H;
    float scale_log2;      // softmax scale times log2(e), > 0
    int causal;            // query i sees keys 0..i (Sq == Sk)
    const uint16_t *Q, *K, *V;
    uint16_t *O;
};
hipError_t launch_attention_fwd(int dtype, const AttnArgs &a, hipStream_t stream);

// Elementwise passes over an M x N matrix: Y = X + bias[n] or Y = GELU_tanh(X)
// (Y may be X).  vec: N % 8 == 0 and X, Y (and bias for the add) 16-byte
// aligned.  At most 8 workgroups per CU (num_cu <= 0: 256 CUs assumed).
enum EwOp { EW_BIAS_ADD = 0, EW_GELU_TANH = 1 };
hipError_t launch_elementwise(int dtype, int op, int64_t M, int N, const uint16_t *bias, const uint16_t *X,
                              uint16_t *Y, bool vec, int num_cu, hipStream_t stream);

}  // namespace tg
