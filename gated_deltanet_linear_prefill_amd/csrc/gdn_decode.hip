// gdn_decode.hip -- batch-1 decode step of the Gated DeltaNet recurrence (t == 1).
//
// "Optimizing on-device inference for Apple Silicon", section "Decode: minimise bytes
// moved per token": at batch 1 the step is bound by the bytes it moves, and the recurrent
// update is fused with its normalisation (here the L2 normalisation of q and k). On
// MI355X the bytes are the fp32 state: every (sequence, V head) state is read from HBM
// once and written back once, with 128-bit coalesced accesses.
//
// One 256-thread workgroup per (sequence, V head) (decode_kernel), or a one-wave workgroup
// per (sequence, V head, block of 32 value channels) when there are too few of those pairs
// to fill the chip (a single sequence; decode_wave_kernel): each channel's update is
// independent, so the blocks need no exchange, and a 32-channel row segment is one whole
// 128-byte line. With the state stored d_k-major (M = S^T,
// M[i][j] = S[j][i]), value channel j is column j of M and evolves on its own:
//   s_k = khat . m_j,  s_q = qhat . m_j,  c_j = beta (v_j - alpha s_k)
//   o_j = alpha s_q + c_j (qhat . khat),   m_j <- alpha m_j + c_j khat
// which is S_t = alpha S_{t-1}(I - beta khat khat^T) + beta v khat^T and o = S_t qhat
// written per column. Thread (rg, cg) holds columns 4cg..4cg+3 of rows rg, rg+RG, ...:
// each load/store instruction of a wave covers whole contiguous rows of M.
#include "gdn_internal.hpp"

namespace gdn {
namespace {

template <int D, int SPLIT>
struct DecodeCfg {
    static constexpr int DC = D / SPLIT;                               // channels per workgroup
    static constexpr int NT = (D * DC / 4 >= 256) ? 256 : D * DC / 4;  // threads
    static constexpr int CG = DC / 4;                                  // float4 per row segment
    static constexpr int RG = NT / CG;                                 // row groups
    static constexpr int RPT = D / RG;                                 // rows per thread
    static constexpr int NW = NT / 64;                                 // waves
    static_assert(RG * RPT == D && CG * RG == NT, "decode tiling");
    static_assert(NT % 64 == 0 && 64 % CG == 0, "a wave holds whole row groups");
};

template <int D, int SPLIT, typename TIn>
__global__ void __launch_bounds__((DecodeCfg<D, SPLIT>::NT))
decode_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
              const float* __restrict__ g, const float* __restrict__ beta,
              const float* state_in, float* __restrict__ out, float* state_out, int h_qk,
              int h_v, float eps)
{
    using Cfg = DecodeCfg<D, SPLIT>;
    constexpr int CG = Cfg::CG, RG = Cfg::RG, RPT = Cfg::RPT, NW = Cfg::NW;
    __shared__ float s_q[D], s_k[D], s_norm[3];
    __shared__ float4 s_part[NW][CG][2];

    const int64_t nh = blockIdx.x / SPLIT;  // sequence * h_v + V head
    const int cb = (int)(blockIdx.x % SPLIT) * Cfg::DC;  // first channel of this workgroup
    const int64_t seq = nh / h_v;
    const int h = (int)(nh - seq * h_v);
    const int hq = h / (h_v / h_qk);
    const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
    const int64_t sbase = nh * (int64_t)D * D + cb;

    // 1. Issue the state loads first: they are the bytes that bound the step.
    float4 m[RPT];
    if (state_in) {
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            m[r] = *reinterpret_cast<const float4*>(state_in + sbase + (int64_t)(rg + RG * r) * D + 4 * cg);
    } else {
#pragma unroll
        for (int r = 0; r < RPT; ++r) m[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // 2. This token's q, k (shared QK head), v slice, gate and write strength.
    const int64_t qk_off = (seq * h_qk + hq) * (int64_t)D;
    if (tid < D) {
        s_q[tid] = load1_f32(q + qk_off + tid);
        s_k[tid] = load1_f32(k + qk_off + tid);
    }
    const float4 vv = load4_f32(v + nh * (int64_t)D + cb + 4 * cg);
    const float alpha = expf(g[nh]);
    const float b = beta[nh];
    __syncthreads();

    // 3. L2 norms and qhat . khat (wave 0), fused here instead of a separate pass.
    if (tid < 64) {
        float qq = 0.f, kk = 0.f, qk = 0.f;
        for (int i = tid; i < D; i += 64) {
            qq += s_q[i] * s_q[i];
            kk += s_k[i] * s_k[i];
            qk += s_q[i] * s_k[i];
        }
        qq = wave_sum(qq);
        kk = wave_sum(kk);
        qk = wave_sum(qk);
        if (tid == 0) {
            const float rq = 1.0f / sqrtf(qq + eps), rk = 1.0f / sqrtf(kk + eps);
            s_norm[0] = rq;
            s_norm[1] = rk;
            s_norm[2] = qk * rq * rk;
        }
    }

    // 4. Partial k . m_j and q . m_j over this thread's rows (raw q, k; scaled below).
    __syncthreads();
    float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const float ki = s_k[rg + RG * r], qi = s_q[rg + RG * r];
        pk.x += ki * m[r].x; pk.y += ki * m[r].y; pk.z += ki * m[r].z; pk.w += ki * m[r].w;
        pq.x += qi * m[r].x; pq.y += qi * m[r].y; pq.z += qi * m[r].z; pq.w += qi * m[r].w;
    }
    // 5. Column sums in a fixed order (so the result is deterministic): first over the row
    // groups of a wave (lanes CG apart hold the same columns) by cross-lane exchanges, then
    // over the waves through LDS.
#pragma unroll
    for (int off = CG; off < 64; off *= 2) {
        pk.x += __shfl_xor(pk.x, off); pk.y += __shfl_xor(pk.y, off);
        pk.z += __shfl_xor(pk.z, off); pk.w += __shfl_xor(pk.w, off);
        pq.x += __shfl_xor(pq.x, off); pq.y += __shfl_xor(pq.y, off);
        pq.z += __shfl_xor(pq.z, off); pq.w += __shfl_xor(pq.w, off);
    }
    const int wave = tid / 64;
    if ((tid & 63) < CG) {
        s_part[wave][cg][0] = pk;
        s_part[wave][cg][1] = pq;
    }
    __syncthreads();
    float4 tk = make_float4(0.f, 0.f, 0.f, 0.f), tq = tk;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const float4 a = s_part[j][cg][0], c = s_part[j][cg][1];
        tk.x += a.x; tk.y += a.y; tk.z += a.z; tk.w += a.w;
        tq.x += c.x; tq.y += c.y; tq.z += c.z; tq.w += c.w;
    }
    const float rq = s_norm[0], rk = s_norm[1], qkh = s_norm[2];
    const float ak = alpha * rk, aq = alpha * rq;
    float4 c;
    c.x = b * (vv.x - ak * tk.x);
    c.y = b * (vv.y - ak * tk.y);
    c.z = b * (vv.z - ak * tk.z);
    c.w = b * (vv.w - ak * tk.w);
    if (rg == 0) {
        float4 o;
        o.x = aq * tq.x + c.x * qkh;
        o.y = aq * tq.y + c.y * qkh;
        o.z = aq * tq.z + c.z * qkh;
        o.w = aq * tq.w + c.w * qkh;
        *reinterpret_cast<float4*>(out + nh * (int64_t)D + cb + 4 * cg) = o;
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const float khi = s_k[rg + RG * r] * rk;
        float4 u;
        u.x = alpha * m[r].x + c.x * khi;
        u.y = alpha * m[r].y + c.y * khi;
        u.z = alpha * m[r].z + c.z * khi;
        u.w = alpha * m[r].w + c.w * khi;
        *reinterpret_cast<float4*>(state_out + sbase + (int64_t)(rg + RG * r) * D + 4 * cg) = u;
    }
}

// One-wave workgroups for launches with fewer than 256 (sequence, V head) pairs (a single
// sequence's layer): such a launch does not fill the chip and the step is bound by latency,
// not bytes. A wave holds a block of DC value channels of one head's state in registers
// (RPT rows per lane), forms the norms itself and sums the columns by cross-lane exchanges,
// so the step needs no workgroup barrier. Same formulas as decode_kernel; the column sums
// are added in another fixed order.
template <int D, int SPLIT>
struct DecodeWaveCfg {
    static constexpr int DC = D / SPLIT;   // channels per workgroup
    static constexpr int CG = DC / 4;      // float4 per row segment
    static constexpr int RG = 64 / CG;     // row groups in the wave
    static constexpr int RPT = D / RG;     // rows per lane
    static constexpr int QPL = D / 64;     // q and k elements per lane
    static_assert(DC % 4 == 0 && 64 % CG == 0 && RG * RPT == D && QPL * 64 == D, "decode wave tiling");
};

template <int D, int SPLIT, typename TIn>
__global__ void __launch_bounds__(64)
decode_wave_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
                   const float* __restrict__ g, const float* __restrict__ beta,
                   const float* state_in, float* __restrict__ out, float* state_out, int h_qk,
                   int h_v, float eps)
{
    using Cfg = DecodeWaveCfg<D, SPLIT>;
    constexpr int CG = Cfg::CG, RG = Cfg::RG, RPT = Cfg::RPT, QPL = Cfg::QPL;
    __shared__ float s_q[D], s_k[D];

    const int64_t nh = blockIdx.x / SPLIT;
    const int cb = (int)(blockIdx.x % SPLIT) * Cfg::DC;
    const int64_t seq = nh / h_v;
    const int h = (int)(nh - seq * h_v);
    const int hq = h / (h_v / h_qk);
    const int l = threadIdx.x, cg = l % CG, rg = l / CG;
    const int64_t sbase = nh * (int64_t)D * D + cb;

    float4 m[RPT];
    if (state_in) {
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            m[r] = *reinterpret_cast<const float4*>(state_in + sbase + (int64_t)(rg + RG * r) * D + 4 * cg);
    } else {
#pragma unroll
        for (int r = 0; r < RPT; ++r) m[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int64_t qk_off = (seq * h_qk + hq) * (int64_t)D;
    float qv[QPL], kv[QPL];
#pragma unroll
    for (int i = 0; i < QPL; ++i) {
        qv[i] = load1_f32(q + qk_off + l + 64 * i);
        kv[i] = load1_f32(k + qk_off + l + 64 * i);
    }
    const float4 vv = load4_f32(v + nh * (int64_t)D + cb + 4 * cg);
    const float alpha = expf(g[nh]);
    const float b = beta[nh];

    float qq = 0.f, kk = 0.f, qk = 0.f;
#pragma unroll
    for (int i = 0; i < QPL; ++i) {
        s_q[l + 64 * i] = qv[i];
        s_k[l + 64 * i] = kv[i];
        qq += qv[i] * qv[i];
        kk += kv[i] * kv[i];
        qk += qv[i] * kv[i];
    }
    qq = wave_sum(qq);
    kk = wave_sum(kk);
    qk = wave_sum(qk);
    const float rq = 1.0f / sqrtf(qq + eps), rk = 1.0f / sqrtf(kk + eps);
    const float qkh = qk * rq * rk;
    __syncthreads();  // one wave: orders its LDS writes before the reads below

    float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const float ki = s_k[rg + RG * r], qi = s_q[rg + RG * r];
        pk.x += ki * m[r].x; pk.y += ki * m[r].y; pk.z += ki * m[r].z; pk.w += ki * m[r].w;
        pq.x += qi * m[r].x; pq.y += qi * m[r].y; pq.z += qi * m[r].z; pq.w += qi * m[r].w;
    }
#pragma unroll
    for (int off = CG; off < 64; off *= 2) {
        pk.x += __shfl_xor(pk.x, off); pk.y += __shfl_xor(pk.y, off);
        pk.z += __shfl_xor(pk.z, off); pk.w += __shfl_xor(pk.w, off);
        pq.x += __shfl_xor(pq.x, off); pq.y += __shfl_xor(pq.y, off);
        pq.z += __shfl_xor(pq.z, off); pq.w += __shfl_xor(pq.w, off);
    }
    const float ak = alpha * rk, aq = alpha * rq;
    float4 c;
    c.x = b * (vv.x - ak * pk.x);
    c.y = b * (vv.y - ak * pk.y);
    c.z = b * (vv.z - ak * pk.z);
    c.w = b * (vv.w - ak * pk.w);
    if (rg == 0) {
        float4 o;
        o.x = aq * pq.x + c.x * qkh;
        o.y = aq * pq.y + c.y * qkh;
        o.z = aq * pq.z + c.z * qkh;
        o.w = aq * pq.w + c.w * qkh;
        *reinterpret_cast<float4*>(out + nh * (int64_t)D + cb + 4 * cg) = o;
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const float khi = s_k[rg + RG * r] * rk;
        float4 u;
        u.x = alpha * m[r].x + c.x * khi;
        u.y = alpha * m[r].y + c.y * khi;
        u.z = alpha * m[r].z + c.z * khi;
        u.w = alpha * m[r].w + c.w * khi;
        *reinterpret_cast<float4*>(state_out + sbase + (int64_t)(rg + RG * r) * D + 4 * cg) = u;
    }
}

template <int D, int SPLIT, typename TIn>
hipError_t launch_decode_wave(const Call& c)
{
    const int64_t blocks = c.n * c.h_v * SPLIT;
    hipLaunchKernelGGL((decode_wave_kernel<D, SPLIT, TIn>), dim3((unsigned)blocks), dim3(64), 0,
                       c.stream, static_cast<const TIn*>(c.q), static_cast<const TIn*>(c.k),
                       static_cast<const TIn*>(c.v), c.g, c.beta, c.state_in, c.out, c.state_out,
                       c.h_qk, c.h_v, c.eps);
    return hipGetLastError();
}

template <int D, int SPLIT, typename TIn>
hipError_t launch_decode_split(const Call& c)
{
    const int64_t blocks = c.n * c.h_v * SPLIT;
    hipLaunchKernelGGL((decode_kernel<D, SPLIT, TIn>), dim3((unsigned)blocks),
                       dim3(DecodeCfg<D, SPLIT>::NT), 0, c.stream, static_cast<const TIn*>(c.q),
                       static_cast<const TIn*>(c.k), static_cast<const TIn*>(c.v), c.g, c.beta,
                       c.state_in, c.out, c.state_out, c.h_qk, c.h_v, c.eps);
    return hipGetLastError();
}

// One workgroup per (sequence, V head); one-wave workgroups of 32 value channels when those
// pairs alone would leave most CUs idle (measured on a 30-layer stack of single-sequence
// steps: 124.9 us per token against 127.2 with 256-thread workgroups of 32 channels and 149
// with one-wave workgroups of 16).
template <int D, typename TIn>
hipError_t launch_decode_t(const Call& c)
{
    if constexpr (D >= 64) {
        if (c.n * c.h_v < 256) return launch_decode_wave<D, D / 32, TIn>(c);
    }
    return launch_decode_split<D, 1, TIn>(c);
}

template <typename TIn>
hipError_t dispatch_d(const Call& c)
{
    switch (c.d) {
        case 16: return launch_decode_t<16, TIn>(c);
        case 32: return launch_decode_t<32, TIn>(c);
        case 64: return launch_decode_t<64, TIn>(c);
        case 128: return launch_decode_t<128, TIn>(c);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const Call& c)
{
    return c.dtype == GDN_BF16 ? dispatch_d<uint16_t>(c) : dispatch_d<float>(c);
}

}  // namespace gdn
