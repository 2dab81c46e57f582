// tg_direct.h -- direct-to-LDS buffer loads (gfx950), shared by every kernel
// that stages operands with them: the tiled GEMM, the M <= 16 kernels and the
// attention forward.
//
// A buffer load with the lds modifier writes each lane's 16 bytes straight
// into LDS (at m0 + instruction offset + 16 * lane) without passing through
// registers.  The loads are written as inline assembly, so the compiler does
// not count them: whoever reads the LDS they fill waits for them with
// wait_vmcnt first (the compiler cannot tell that the LDS they write is not
// the LDS being read, and would otherwise wait for every load in flight
// before each use of LDS data).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {
namespace direct {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource words for the inline-asm load: base, stride 0, byte range,
// word 3 of the gfx9 family (32-bit data format).  Loads beyond the range
// write zeros to LDS.
__device__ __forceinline__ i32x4 rsrc_words(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, 0x00020000};
}

// The 32-bit LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_address(const void *q) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)q;
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

// dma16 with a wave-uniform byte offset in an SGPR (the instruction's
// soffset), added to every lane's address without a vector add.  Whether the
// range check of the buffer covers soffset is not relied on: a caller passes
// it only where voffset + soffset + OFF lies inside the buffer for every lane
// whose voffset + OFF does, and gives a lane that must read zeros a voffset
// of 2^31 or more (with voffset + soffset + OFF still below 2^32).
template <int OFF>
__device__ __forceinline__ void dma16s(const i32x4 &rsrc, uint32_t voffset, uint32_t soffset, uint32_t m0) {
    static_assert(OFF >= 0 && OFF < 4096, "12-bit instruction offset");
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%4 lds" ::"v"(voffset), "s"(rsrc), "s"(soffset),
                 "{m0}"(m0), "i"(OFF));
}

// dma16 with the instruction offset 1024 rq (rq = 0..3, a compile-time value
// after unrolling): loads of one 4 KB block share m0.
__device__ __forceinline__ void dma16_rq(int rq, const i32x4 &rsrc, uint32_t voffset, uint32_t m0) {
    switch (rq) {
    case 0: dma16<0>(rsrc, voffset, m0); break;
    case 1: dma16<1024>(rsrc, voffset, m0); break;
    case 2: dma16<2048>(rsrc, voffset, m0); break;
    default: dma16<3072>(rsrc, voffset, m0); break;
    }
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

}  // namespace direct
}  // namespace tg
