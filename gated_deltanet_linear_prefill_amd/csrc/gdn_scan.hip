// gdn_scan.hip -- direct-scan prefill of the Gated DeltaNet recurrence.
//
// "Optimizing on-device inference for Apple Silicon", section "Keep the recurrent state
// on-chip": each column of the state goes to one SIMD group, split across its lanes'
// registers, loaded once, carried through the whole scan and written back once; partial
// results are exchanged with cross-lane operations rather than shared memory. The same
// idea on CDNA4: a value channel j is column j of M = S^T (d_k long); it lives in the
// VGPRs of one 16-lane DPP row (d_k/16 rows per lane), and its two dot products per token
// are summed across that row with four DPP adds each. A wave holds 4 columns, a
// workgroup 16.
//
// Per token and column, with khat/qhat normalised and qk = qhat . khat:
//   s_k = khat . m_j,  s_q = qhat . m_j,  c = beta (v_j - alpha s_k)
//   o_j = alpha s_q + c qk,                m_j <- alpha m_j + c khat
// i.e. S_t = alpha S_{t-1}(I - beta khat khat^T) + beta v khat^T, o_t = S_t qhat, by column.
//
// A first small kernel writes qhat, khat (fp32) and qk per (token, QK head) to the
// workspace, so the scan itself spends its VALU cycles on the state only.
#include "gdn_internal.hpp"

namespace gdn {
namespace {

size_t align256(size_t x)
{
    return (x + 255) & ~size_t(255);
}

// ------------------------------------------------------------------ q/k normalisation
// One 16-lane row per (sequence, token, QK head): qhat = q / sqrt(sum q^2 + eps), khat
// likewise, qk = qhat . khat (from the raw dot product and both scales).
template <int D, typename TIn>
__global__ void __launch_bounds__(256)
qk_normalise_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, int64_t rows, float eps,
                    float* __restrict__ qhat, float* __restrict__ khat, float* __restrict__ qkdot)
{
    constexpr int RPL = D / 16;
    const int sub = threadIdx.x & 15;
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int64_t r = row < rows ? row : rows - 1;  // all lanes stay active for the DPP sums
    float qv[RPL], kv[RPL];
    load_n<RPL>(q + r * D + sub * RPL, qv);
    load_n<RPL>(k + r * D + sub * RPL, kv);
    float qq = 0.f, kk = 0.f, qk = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        qq += qv[i] * qv[i];
        kk += kv[i] * kv[i];
        qk += qv[i] * kv[i];
    }
    qq = row16_sum(qq);
    kk = row16_sum(kk);
    qk = row16_sum(qk);
    const float rq = 1.0f / sqrtf(qq + eps), rk = 1.0f / sqrtf(kk + eps);
    if (row < rows) {
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            qhat[r * D + sub * RPL + i] = qv[i] * rq;
            khat[r * D + sub * RPL + i] = kv[i] * rk;
        }
        if (sub == 0) qkdot[r] = qk * rq * rk;
    }
}

// ------------------------------------------------------------------ the scan
template <int RPL>
struct Tok {
    float k[RPL], q[RPL];
    float v, g, b, qk;
};

template <int D, typename TIn>
__global__ void __launch_bounds__(256)
scan_kernel(const float* __restrict__ qhat, const float* __restrict__ khat,
            const float* __restrict__ qkdot, const TIn* __restrict__ v, const float* __restrict__ g,
            const float* __restrict__ beta, const float* state_in, float* __restrict__ out,
            float* state_out, int64_t T, int h_qk, int h_v)
{
    constexpr int RPL = D / 16;  // state rows per lane
    constexpr int NCB = D / 16;  // 16-column blocks per head
    constexpr int ST = 4;        // tokens per pipeline stage

    // Workgroups that share a QK head's normalised rows (its V heads' column blocks, which
    // are consecutive in `lin`) run on one XCD (blockIdx % 8 picks the XCD), so those rows
    // are fetched into one L2 rather than into all eight.
    int64_t lin = blockIdx.x;
    if (gridDim.x % 8 == 0) lin = (int64_t)(blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
    const int64_t nh = lin / NCB;  // sequence * h_v + V head
    const int cb = (int)(lin % NCB);
    const int64_t seq = nh / h_v;
    const int h = (int)(nh - seq * h_v);
    const int hq = h / (h_v / h_qk);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane & 15;
    const int j = cb * 16 + wave * 4 + (lane >> 4);  // this lane's value channel
    const int row0 = sub * RPL;                       // first state row of this lane

    float m[RPL];
    const int64_t sbase = nh * (int64_t)D * D;
#pragma unroll
    for (int r = 0; r < RPL; ++r)
        m[r] = state_in ? state_in[sbase + (int64_t)(row0 + r) * D + j] : 0.f;

    auto load_tok = [&](Tok<RPL>& x, int64_t tt) {
        tt = tt < T ? tt : T - 1;  // clamped: a tail stage reads valid memory it never uses
        const int64_t qrow = (seq * T + tt) * h_qk + hq;
        const int64_t vrow = (seq * T + tt) * h_v + h;
        load_n<RPL>(khat + qrow * D + row0, x.k);
        load_n<RPL>(qhat + qrow * D + row0, x.q);
        x.qk = qkdot[qrow];
        x.v = load1_f32(v + vrow * D + j);
        x.g = g[vrow];
        x.b = beta[vrow];
    };

    float obuf = 0.f;  // lane `sub` keeps the output of token (16-block base + sub)
    auto step = [&](const Tok<RPL>& x, int64_t tt) {
        float sk0 = 0.f, sk1 = 0.f, sq0 = 0.f, sq1 = 0.f;
#pragma unroll
        for (int r = 0; r < RPL; r += 2) {
            sk0 += x.k[r] * m[r];
            sq0 += x.q[r] * m[r];
            if (r + 1 < RPL) {
                sk1 += x.k[r + 1] * m[r + 1];
                sq1 += x.q[r + 1] * m[r + 1];
            }
        }
        const float sk = row16_sum(sk0 + sk1);
        const float sq = row16_sum(sq0 + sq1);
        const float alpha = expf(x.g);
        const float c = x.b * (x.v - alpha * sk);
        const float o = alpha * sq + c * x.qk;
#pragma unroll
        for (int r = 0; r < RPL; ++r) m[r] = alpha * m[r] + c * x.k[r];
        const int u = (int)(tt & 15);
        obuf = (sub == u) ? o : obuf;
        if (u == 15 || tt == T - 1) {
            const int64_t t_out = (tt & ~int64_t(15)) + sub;
            if (t_out <= tt) out[((seq * T + t_out) * h_v + h) * D + j] = obuf;
        }
    };

    Tok<RPL> A[ST], B[ST];
#pragma unroll
    for (int s = 0; s < ST; ++s) load_tok(A[s], s);
    for (int64_t t0 = 0; t0 < T; t0 += 2 * ST) {
#pragma unroll
        for (int s = 0; s < ST; ++s) load_tok(B[s], t0 + ST + s);
#pragma unroll
        for (int s = 0; s < ST; ++s)
            if (t0 + s < T) step(A[s], t0 + s);
#pragma unroll
        for (int s = 0; s < ST; ++s) load_tok(A[s], t0 + 2 * ST + s);
#pragma unroll
        for (int s = 0; s < ST; ++s)
            if (t0 + ST + s < T) step(B[s], t0 + ST + s);
    }

#pragma unroll
    for (int r = 0; r < RPL; ++r) state_out[sbase + (int64_t)(row0 + r) * D + j] = m[r];
}

struct ScanWs {
    size_t qhat, khat, qk, total;
};

ScanWs scan_ws_layout(int64_t n, int64_t t, int32_t h_qk, int32_t d)
{
    const size_t rows = (size_t)n * (size_t)t * (size_t)h_qk;
    ScanWs w;
    w.qhat = 0;
    w.khat = align256(rows * d * sizeof(float));
    w.qk = w.khat + align256(rows * d * sizeof(float));
    w.total = w.qk + align256(rows * sizeof(float));
    return w;
}

template <int D, typename TIn>
hipError_t launch_scan_t(const Call& c)
{
    const ScanWs w = scan_ws_layout(c.n, c.t, c.h_qk, D);
    char* ws = static_cast<char*>(c.ws);
    float* qhat = reinterpret_cast<float*>(ws + w.qhat);
    float* khat = reinterpret_cast<float*>(ws + w.khat);
    float* qk = reinterpret_cast<float*>(ws + w.qk);
    const int64_t rows = c.n * c.t * c.h_qk;
    hipLaunchKernelGGL((qk_normalise_kernel<D, TIn>), dim3((unsigned)((rows + 15) / 16)), dim3(256),
                       0, c.stream, static_cast<const TIn*>(c.q), static_cast<const TIn*>(c.k),
                       rows, c.eps, qhat, khat, qk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t blocks = c.n * c.h_v * (D / 16);
    hipLaunchKernelGGL((scan_kernel<D, TIn>), dim3((unsigned)blocks), dim3(256), 0, c.stream, qhat,
                       khat, qk, static_cast<const TIn*>(c.v), c.g, c.beta, c.state_in, c.out,
                       c.state_out, c.t, c.h_qk, c.h_v);
    return hipGetLastError();
}

// The ablation of state residency: the same normalisation and scan kernels, but the scan is
// launched once per block of block_t tokens of each sequence, so the state leaves the chip
// after every block (written to state_out, read back by the next block's launch).
template <int D, typename TIn>
hipError_t launch_scan_blockwise_t(const Call& c, int64_t block_t)
{
    const ScanWs w = scan_ws_layout(c.n, c.t, c.h_qk, D);
    char* ws = static_cast<char*>(c.ws);
    const float* qhat = reinterpret_cast<const float*>(ws + w.qhat);
    const float* khat = reinterpret_cast<const float*>(ws + w.khat);
    const float* qk = reinterpret_cast<const float*>(ws + w.qk);
    const int64_t rows = c.n * c.t * c.h_qk;
    hipLaunchKernelGGL((qk_normalise_kernel<D, TIn>), dim3((unsigned)((rows + 15) / 16)), dim3(256),
                       0, c.stream, static_cast<const TIn*>(c.q), static_cast<const TIn*>(c.k),
                       rows, c.eps, reinterpret_cast<float*>(ws + w.qhat),
                       reinterpret_cast<float*>(ws + w.khat), reinterpret_cast<float*>(ws + w.qk));
    hipError_t e = hipGetLastError();
    const TIn* v = static_cast<const TIn*>(c.v);
    const int64_t state_elems = (int64_t)c.h_v * D * D;
    for (int64_t s = 0; s < c.n && e == hipSuccess; ++s) {
        for (int64_t t0 = 0; t0 < c.t && e == hipSuccess; t0 += block_t) {
            const int64_t len = c.t - t0 < block_t ? c.t - t0 : block_t;
            const int64_t tok = s * c.t + t0;
            const float* si = t0 == 0 ? (c.state_in ? c.state_in + s * state_elems : nullptr)
                                      : c.state_out + s * state_elems;
            hipLaunchKernelGGL((scan_kernel<D, TIn>), dim3((unsigned)(c.h_v * (D / 16))), dim3(256), 0,
                               c.stream, qhat + tok * c.h_qk * D, khat + tok * c.h_qk * D,
                               qk + tok * c.h_qk, v + tok * c.h_v * D, c.g + tok * c.h_v,
                               c.beta + tok * c.h_v, si, c.out + tok * c.h_v * D,
                               c.state_out + s * state_elems, len, c.h_qk, c.h_v);
            e = hipGetLastError();
        }
    }
    return e;
}

template <typename TIn>
hipError_t dispatch_d(const Call& c)
{
    switch (c.d) {
        case 16: return launch_scan_t<16, TIn>(c);
        case 32: return launch_scan_t<32, TIn>(c);
        case 64: return launch_scan_t<64, TIn>(c);
        case 128: return launch_scan_t<128, TIn>(c);
        default: return hipErrorInvalidValue;
    }
}

template <typename TIn>
hipError_t dispatch_blockwise(const Call& c, int64_t block_t)
{
    switch (c.d) {
        case 16: return launch_scan_blockwise_t<16, TIn>(c, block_t);
        case 32: return launch_scan_blockwise_t<32, TIn>(c, block_t);
        case 64: return launch_scan_blockwise_t<64, TIn>(c, block_t);
        case 128: return launch_scan_blockwise_t<128, TIn>(c, block_t);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t scan_workspace_bytes(int64_t n, int64_t t, int32_t h_qk, int32_t h_v, int32_t d)
{
    (void)h_v;
    return scan_ws_layout(n, t, h_qk, d).total;
}

hipError_t launch_scan(const Call& c)
{
    return c.dtype == GDN_BF16 ? dispatch_d<uint16_t>(c) : dispatch_d<float>(c);
}

hipError_t launch_scan_blockwise(const Call& c, int64_t block_t)
{
    return c.dtype == GDN_BF16 ? dispatch_blockwise<uint16_t>(c, block_t)
                               : dispatch_blockwise<float>(c, block_t);
}

}  // namespace gdn
