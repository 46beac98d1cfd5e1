// gdn_internal.hpp -- shared host/device pieces of libgdn.so (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// A validated call: sizes checked, pointers non-null where required, aligned, disjoint.
struct Call {
    int64_t n, t;
    int32_t h_qk, h_v, d;
    int32_t dtype;  // gdn_dtype of q, k, v
    float eps;
    const void *q, *k, *v;
    const float *g, *beta, *state_in;
    float *out, *state_out;
    void* ws;
    size_t ws_bytes;
    hipStream_t stream;
};

// Kernel launchers, one per translation unit. Each returns hipGetLastError() after its
// launches. The caller has validated everything the kernels assume.
hipError_t launch_decode(const Call& c);
hipError_t launch_scan(const Call& c);
hipError_t launch_scan_blockwise(const Call& c, int64_t block_t);  // block_t > 0
// parts: kChunkPrep (the per-chunk preparation into the workspace), kChunkScan (the
// sequential pass that reads it), or both; the scan must follow a prep of the same call.
constexpr int kChunkPrep = 1, kChunkScan = 2;
hipError_t launch_chunked(const Call& c, int chunk, int parts = kChunkPrep | kChunkScan);
hipError_t launch_state_passthrough(const Call& c);  // t == 0: state_out = state_in or 0
hipError_t launch_mfma_loop(int64_t iters, int32_t blocks, float* sink, hipStream_t stream);
hipError_t launch_lds_fill(uint32_t pattern, int32_t blocks, uint32_t* sink, hipStream_t stream);
hipError_t launch_stream_copy(const void* src, void* dst, int64_t n16, int32_t blocks,
                              hipStream_t stream);

size_t scan_workspace_bytes(int64_t n, int64_t t, int32_t h_qk, int32_t h_v, int32_t d);
size_t chunked_workspace_bytes(int64_t n, int64_t t, int32_t h_qk, int32_t h_v, int32_t d,
                               int chunk, int32_t dtype);

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16)
{
    return __uint_as_float(bits16 << 16);
}

// Four consecutive q/k/v elements as fp32 (an 8-byte load for bf16, 16 bytes for fp32).
template <typename TIn>
__device__ __forceinline__ float4 load4_f32(const TIn* p);

template <>
__device__ __forceinline__ float4 load4_f32<float>(const float* p)
{
    return *reinterpret_cast<const float4*>(p);
}

template <>
__device__ __forceinline__ float4 load4_f32<uint16_t>(const uint16_t* p)
{
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(bf16_bits_to_f32(u.x & 0xffffu), bf16_bits_to_f32(u.x >> 16),
                       bf16_bits_to_f32(u.y & 0xffffu), bf16_bits_to_f32(u.y >> 16));
}

template <typename TIn>
__device__ __forceinline__ float load1_f32(const TIn* p);

template <>
__device__ __forceinline__ float load1_f32<float>(const float* p)
{
    return *p;
}

template <>
__device__ __forceinline__ float load1_f32<uint16_t>(const uint16_t* p)
{
    return bf16_bits_to_f32(*p);
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane receives the same (bitwise) total.
__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    x += dpp_f<0x141>(x);  // row_half_mirror: lane i <-> 7 - i within 8
    x += dpp_f<0x140>(x);  // row_mirror: lane i <-> 15 - i within 16
    return x;
}

// Buffer resources: a base address and byte range in scalar registers, re-based once per
// chunk with scalar adds, while each lane keeps fixed byte offsets. Lanes whose offset
// falls outside the range read zero (and their stores are dropped), which handles the rows
// past the end of a sequence and padded features without per-lane branches. The 0x00020000
// word is the raw (untyped, unswizzled) descriptor format of the gfx9 family.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes)
{
    const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

// A byte offset beyond every buffer range used here (ranges stay below 2^30; the host
// checks the chunk's q/k/v/out extents against that bound). Added to an in-range offset
// (below 2^30) it stays below 2^32, so the hardware's unsigned offset does not wrap.
constexpr uint32_t OOR = 0x60000000u;

// Loads that write LDS directly: each lane's 16 (load_to_lds) or 4 (load_to_lds4) bytes at
// byte offset `off` of the buffer land in LDS at `lds` + 16 (or 4) * lane; `lds` is the same
// for the whole wave. Lanes whose offset is out of range write zeros.
__device__ __forceinline__ void load_to_lds(__amdgpu_buffer_rsrc_t r, void* lds, int off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}

__device__ __forceinline__ void load_to_lds4(__amdgpu_buffer_rsrc_t r, void* lds, int off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, off, 0, 0, 0);
}

template <int N, typename TIn>
__device__ __forceinline__ void load_n(const TIn* p, float* x)
{
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const float4 a = load4_f32(p + i);
            x[i] = a.x; x[i + 1] = a.y; x[i + 2] = a.z; x[i + 3] = a.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = load1_f32(p + i);
    }
}

}  // namespace gdn
