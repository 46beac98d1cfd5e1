// gdn_calib.hip -- calibration kernels (measurement only; the prefill and decode paths never
// call them):
//  * a loop of dense bf16 MFMAs, for the achievable matrix rate that the chunked kernels'
//    MFMA use is reported against;
//  * a streaming device copy, for the achievable HBM rate (read + write) that the decode
//    step, which reads and writes every state element once, is reported against;
//  * an LDS fill (diagnostic): workgroups that take a CU's whole LDS and fill it with one
//    32-bit pattern, so that a kernel launched after it that reads LDS it never wrote sees
//    that pattern (a NaN, say) rather than whatever the previous kernel left there.
//
// Each wave keeps four independent 32x32x16 accumulators, so consecutive MFMAs never wait
// for each other, and writes one sum per lane at the end so that nothing is optimised away.
// (On gfx950 the 32x32x16 bf16 form sustains about 2.0 PFLOP/s in such a loop, the 16x16x32
// form about 1.2-1.4: measured, the former is the achievable figure.)
#include "gdn_internal.hpp"

namespace gdn {
namespace {

typedef __bf16 calib_bf16x8 __attribute__((ext_vector_type(8)));
typedef float calib_floatx16 __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) mfma_loop_kernel(int64_t iters, float* __restrict__ sink)
{
    const int l = threadIdx.x & 63;
    calib_bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(l + i));
        b[i] = (__bf16)(0.002f * (float)(l - i));
    }
    calib_floatx16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Streaming copy: every thread moves one 16-byte element per iteration (load, then store)
// over a grid-stride loop, so that at any time the whole grid works in one narrow address
// window and loads and stores of different waves are in flight together. Of the forms
// measured on MI355X (one to eight elements per thread per iteration, 256 to 8192
// workgroups, and a tile-per-workgroup copy shaped like the decode step), this one with 1024
// workgroups moved the most bytes per second, warm and with the buffers out of the MALL.
__global__ void __launch_bounds__(256) stream_copy_kernel(const float4* __restrict__ src,
                                                          float4* __restrict__ dst, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

// 160 KB of LDS per workgroup: the whole of a CU's LDS, so one workgroup per CU at a time.
constexpr int kFillLdsBytes = 160 * 1024;

__global__ void __launch_bounds__(256) lds_fill_kernel(uint32_t pattern, uint32_t* __restrict__ sink)
{
    __shared__ __align__(16) uint32_t s_fill[kFillLdsBytes / 4];
    for (int i = threadIdx.x; i < kFillLdsBytes / 4; i += 256) s_fill[i] = pattern;
    __syncthreads();
    // one read back, so that the stores are kept
    if (threadIdx.x == 0 && s_fill[(blockIdx.x * 977u) % (kFillLdsBytes / 4)] != pattern) sink[0] = 1u;
}

}  // namespace

hipError_t launch_lds_fill(uint32_t pattern, int32_t blocks, uint32_t* sink, hipStream_t stream)
{
    hipLaunchKernelGGL(lds_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, pattern, sink);
    return hipGetLastError();
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t n16, int32_t blocks,
                              hipStream_t stream)
{
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const float4*>(src), static_cast<float4*>(dst), n16);
    return hipGetLastError();
}

hipError_t launch_mfma_loop(int64_t iters, int32_t blocks, float* sink, hipStream_t stream)
{
    hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, iters, sink);
    return hipGetLastError();
}

}  // namespace gdn
