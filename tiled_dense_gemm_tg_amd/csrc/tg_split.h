// tg_split.h -- the cross-workgroup step of split-K in the M <= 16 kernels.
//
// Several workgroups compute partial sums of the same 16 x 64 output block
// over parts of the K range (an even split of every block's K range, or the
// stream-K ranges of the skinny kernel).  Each publishes its partial block
// to the workspace and counts itself in the block's counter; the last to
// arrive reads every part, adds them in K order (so the sum does not depend
// on which workgroup came last), finishes the block and resets the counter
// to zero.  No workgroup ever waits for another, so no schedule of the
// workgroups can deadlock.
//
// Visibility without cache-wide fences: the partials are stored and loaded
// at device scope (sc1: written through to, and read from, the level all
// CUs share, never a stale copy in one XCD's L2), each wave waits for its
// stores to complete before the workgroup barrier that precedes the counter
// update, and the partial loads are issued only after the counter update
// has returned.
#pragma once

#include "tg_device.h"
#include "tg_launch.h"

namespace tg {

constexpr int CPOL_SC1 = 16;   // cache policy of a buffer access: device scope

// The partial blocks of one 16 x 64 output block: `nparts` of 1024 floats
// from `part`.  Waves 0..3 of a workgroup hold in y its sums for column
// group `group` (= wave) of every lane: values 4 (64 group + lane) .. + 3 of
// a partial block.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(float *part, int nparts) {
    return __builtin_amdgcn_make_buffer_rsrc(part, (short)0, nparts * 4096, 0x00020000);
}

// Stores the workgroup's partial block at slot `mine`, at device scope
// (waves 0..3).  Does not wait for the store to complete.
__device__ __forceinline__ void part_publish(float *part, int nparts, int mine, const float (&y)[4], int group) {
    const int lane = threadIdx.x & 63;
    const uint32_t off = 16u * (uint32_t)(64 * group + lane);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{y[0], y[1], y[2], y[3]}),
                                           part_rsrc(part, nparts), (int)(off + 4096u * (uint32_t)mine), 0, CPOL_SC1);
}

// y = the sum of the nparts partial blocks in slot order (waves 0..3), eight
// in flight at a time; reads past the last slot are out of range and give
// +0, which changes no sum (y starts at +0 and so is never -0).
__device__ __forceinline__ void part_sum(float *part, int nparts, float (&y)[4], int group) {
    const int lane = threadIdx.x & 63;
    const uint32_t off = 16u * (uint32_t)(64 * group + lane);
    const __amdgpu_buffer_rsrc_t rp = part_rsrc(part, nparts);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        y[j] = 0.f;
    for (int q0 = 0; q0 < nparts; q0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t o = q0 + i < nparts ? off + 4096u * (uint32_t)(q0 + i) : 0xFFFFFFF0u;
            // the whole vector is reinterpreted: clang's __builtin_bit_cast
            // of one element of a vector reads element 0
            v[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, (int)o, 0, CPOL_SC1));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                y[j] += v[i][j];
    }
}

// Counts one arrival in `count` (one thread); true for the last of nparts,
// which also leaves the counter zero for the next call.
__device__ __forceinline__ bool part_arrive(uint32_t *count, int nparts) {
    const uint32_t before = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = before == (uint32_t)(nparts - 1);
    if (last)
        __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return last;
}

// Called by every wave of the workgroup (it holds barriers): publishes the
// partial at slot `mine`, waits for it, counts the arrival.  Returns true in
// waves 0..3 of the last workgroup to arrive, with y then holding the sum of
// every partial in slot order; false everywhere else (those waves have
// nothing more to do for this block).
__device__ __forceinline__ bool part_exchange(float *part, uint32_t *count, int nparts, int mine, float (&y)[4],
                                              int group) {
    __shared__ uint32_t is_last;
    const int wave = threadIdx.x >> 6;
    if (wave < 4) {
        part_publish(part, nparts, mine, y, group);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (threadIdx.x == 0)
        is_last = part_arrive(count, nparts);
    __syncthreads();
    if (!is_last || wave >= 4)
        return false;
    part_sum(part, nparts, y, group);
    return true;
}

// Even split-K: block `blk` has ws.splits partials, in split order, and
// this workgroup is split `split` of it.
__device__ __forceinline__ bool split_exchange(const SplitWs &ws, int64_t blk, int split, float (&y)[4], int group) {
    return part_exchange(ws.part + blk * ws.splits * 1024, ws.count + blk, ws.splits, split, y, group);
}

}  // namespace tg
