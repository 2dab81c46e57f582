// tg_split.h -- the cross-workgroup step of split-K in the M <= 16 kernels.
//
// With splits > 1 several workgroups compute partial sums of the same 16 x 64
// output block over parts of the K range.  Each publishes its partial block
// to the workspace and counts itself in the block's counter; the last to
// arrive reads every split's partial, adds them in split order (so the sum
// does not depend on which workgroup came last), finishes the block and
// resets the counter to zero.  No workgroup ever waits for another, so no
// schedule of the workgroups can deadlock.
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

// Called by every wave of the workgroup (it holds barriers).  Waves 0..3
// hold in y the workgroup's sums for column group `group` (= wave) of every
// lane: values 4 (64 group + lane) .. + 3 of the 1024-value partial block.
// Returns true in waves 0..3 of the last workgroup of block `blk` to arrive,
// with y then holding the sum over every split; false everywhere else (those
// waves have nothing more to do).
__device__ __forceinline__ bool split_exchange(const SplitWs &ws, int64_t blk, int split, float (&y)[4], int group) {
    __shared__ uint32_t is_last;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int splits = ws.splits;
    const __amdgpu_buffer_rsrc_t rp =
        __builtin_amdgcn_make_buffer_rsrc(ws.part + blk * splits * 1024, (short)0, splits * 4096, 0x00020000);
    const uint32_t off = 16u * (uint32_t)(64 * group + lane);
    if (wave < 4) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{y[0], y[1], y[2], y[3]}), rp,
                                               (int)(off + 4096u * (uint32_t)split), 0, CPOL_SC1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (tid == 0) {
        const uint32_t before = __hip_atomic_fetch_add(ws.count + blk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = before == (uint32_t)(splits - 1);
        if (is_last)   // every split has counted: leave the counter zero for the next call
            __hip_atomic_store(ws.count + blk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!is_last || wave >= 4)
        return false;
    // eight partials in flight at a time, added in split order; reads past
    // the last split are out of range and give +0, which changes no sum (y
    // starts at +0 and so is never -0)
#pragma unroll
    for (int j = 0; j < 4; ++j)
        y[j] = 0.f;
    for (int q0 = 0; q0 < splits; q0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t o = q0 + i < splits ? off + 4096u * (uint32_t)(q0 + i) : 0xFFFFFFF0u;
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
    return true;
}

}  // namespace tg
