// elementwise.hip -- the epilogue steps as separate passes over C in HBM:
// y = x + bias[n] and y = GELU_tanh(x), each reading and writing a whole M x N
// matrix of 16-bit values.  Run after a GEMM without epilogue they form the
// unfused three-launch baseline that the fourth TileLang page ("Designing
// high-performance GPU kernels with TileLang", part 3 "Epilogue fusion")
// compares the fused epilogue against; the fused path applies the same
// arithmetic (tg_device.h) to the fp32 accumulator instead, with one rounding.
//
// Both passes are HBM-bound (4 bytes moved per element, one or a few ALU
// operations), so the layout of the work is about streaming: with N % 8 == 0
// and 16-byte aligned operands each lane moves whole 16-byte chunks (8
// elements of one row), several chunks in flight per lane, over a grid sized
// to a few workgroups per CU; otherwise one element per lane.
#include "tg_device.h"
#include "tg_launch.h"

namespace tg {
namespace {

constexpr int NTHREADS = 256;
constexpr int UNR = 4;            // 16-byte chunks in flight per lane

template <class T, int OP>
__device__ __forceinline__ uint16_t apply(uint16_t x, float b) {
    const float v = T::to_f32(x);
    if constexpr (OP == EW_BIAS_ADD)
        return T::from_f32(v + b);
    else
        return T::from_f32(gelu_tanh(v));
}

// 8 elements per chunk; chunk c covers elements 8c .. 8c+7 of one row
// (N % 8 == 0).  Every index used is below `chunks`.
template <class T, int OP>
__global__ __launch_bounds__(NTHREADS) void ew_vec_kernel(int64_t chunks, int N, const uint16_t *__restrict__ bias,
                                                         const uint16_t *X, uint16_t *Y) {
    const u32x4 *x4 = reinterpret_cast<const u32x4 *>(X);
    u32x4 *y4 = reinterpret_cast<u32x4 *>(Y);
    const int64_t stride = (int64_t)gridDim.x * NTHREADS;
    for (int64_t c0 = (int64_t)blockIdx.x * NTHREADS + threadIdx.x; c0 < chunks; c0 += stride * UNR) {
        u32x4 v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int64_t c = c0 + u * stride;
            if (c < chunks)
                v[u] = x4[c];
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int64_t c = c0 + u * stride;
            if (c >= chunks)
                continue;
            float b[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if constexpr (OP == EW_BIAS_ADD) {
                const int n = (int)((c * 8) % N);
                const u32x4 bb = *reinterpret_cast<const u32x4 *>(bias + n);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    b[2 * q] = T::to_f32((uint16_t)(bb[q] & 0xffff));
                    b[2 * q + 1] = T::to_f32((uint16_t)(bb[q] >> 16));
                }
            }
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = pack2(apply<T, OP>((uint16_t)(v[u][q] & 0xffff), b[2 * q]),
                             apply<T, OP>((uint16_t)(v[u][q] >> 16), b[2 * q + 1]));
            y4[c] = o;
        }
    }
}

template <class T, int OP>
__global__ __launch_bounds__(NTHREADS) void ew_scalar_kernel(int64_t total, int N, const uint16_t *__restrict__ bias,
                                                            const uint16_t *X, uint16_t *Y) {
    const int64_t stride = (int64_t)gridDim.x * NTHREADS;
    for (int64_t i = (int64_t)blockIdx.x * NTHREADS + threadIdx.x; i < total; i += stride) {
        float b = 0.f;
        if constexpr (OP == EW_BIAS_ADD)
            b = T::to_f32(bias[i % N]);
        Y[i] = apply<T, OP>(X[i], b);
    }
}

template <class T, int OP>
hipError_t launch_typed(int64_t M, int N, const uint16_t *bias, const uint16_t *X, uint16_t *Y, bool vec,
                        int num_cu, hipStream_t stream) {
    const int64_t total = M * (int64_t)N;
    const int64_t units = vec ? total / 8 : total;
    const int64_t cap = (int64_t)(num_cu > 0 ? num_cu : 256) * 8;
    const int64_t need = (units + (int64_t)NTHREADS * (vec ? UNR : 1) - 1) / ((int64_t)NTHREADS * (vec ? UNR : 1));
    const int grid = (int)(need < cap ? (need > 0 ? need : 1) : cap);
    if (vec)
        hipLaunchKernelGGL((ew_vec_kernel<T, OP>), dim3(grid), dim3(NTHREADS), 0, stream, units, N, bias, X, Y);
    else
        hipLaunchKernelGGL((ew_scalar_kernel<T, OP>), dim3(grid), dim3(NTHREADS), 0, stream, units, N, bias, X, Y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_elementwise(int dtype, int op, int64_t M, int N, const uint16_t *bias, const uint16_t *X,
                              uint16_t *Y, bool vec, int num_cu, hipStream_t stream) {
    if (dtype == 0)
        return op == EW_BIAS_ADD ? launch_typed<F16, EW_BIAS_ADD>(M, N, bias, X, Y, vec, num_cu, stream)
                                 : launch_typed<F16, EW_GELU_TANH>(M, N, bias, X, Y, vec, num_cu, stream);
    return op == EW_BIAS_ADD ? launch_typed<BF16, EW_BIAS_ADD>(M, N, bias, X, Y, vec, num_cu, stream)
                             : launch_typed<BF16, EW_GELU_TANH>(M, N, bias, X, Y, vec, num_cu, stream);
}

}  // namespace tg
