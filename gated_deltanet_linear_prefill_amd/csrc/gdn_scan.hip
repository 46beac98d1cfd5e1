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
// A first small kernel writes qhat, khat (fp32) and qk per (token, QK head), and the decay
// alpha = exp(g) per (token, V head), to the workspace, so the scan itself spends its VALU
// cycles on the state only; the scan reads them through LDS, staged well ahead of use.
#include "gdn_internal.hpp"

namespace gdn {
namespace {

size_t align256(size_t x)
{
    return (x + 255) & ~size_t(255);
}

// ------------------------------------------------------------------ q/k normalisation
// One 16-lane row per (sequence, token, QK head): qhat = q / sqrt(sum q^2 + eps), khat
// likewise, qk = qhat . khat (from the raw dot product and both scales); and the decay
// alpha = exp(g) of the QK head's V heads at that token.
template <int D, typename TIn>
__global__ void __launch_bounds__(256)
qk_normalise_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const float* __restrict__ g,
                    int64_t rows, int h_qk, int h_v, float eps, float* __restrict__ qhat,
                    float* __restrict__ khat, float* __restrict__ qkdot, float* __restrict__ alpha)
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
        const int grp = h_v / h_qk;
        const int64_t tok = r / h_qk;
        const int hv0 = (int)(r - tok * h_qk) * grp;
        for (int i = sub; i < grp; i += 16) alpha[tok * h_v + hv0 + i] = expf(g[tok * h_v + hv0 + i]);
    }
}

// ------------------------------------------------------------------ the scan
// The inputs of each token (qhat and khat rows of the QK head, alpha, beta, qk and the
// workgroup's 16 value channels) reach LDS by loads that write it directly, in stages of
// SCAN_ST tokens, three stages ahead of use, into a ring of SCAN_NSL stages: the loads of a
// stage are spread evenly over the four waves, and each wave waits for them with an exact
// count, since per stage it issues the same number of vector memory operations (its share
// of the loads, and one store of the stage's outputs).
constexpr int SCAN_ST = 16;  // tokens per stage
constexpr int SCAN_NSL = 4;  // stages in the ring

template <int D, typename TIn>
__global__ void __launch_bounds__(256)
scan_kernel(const float* __restrict__ qhat, const float* __restrict__ khat,
            const float* __restrict__ qkdot, const float* __restrict__ alpha,
            const TIn* __restrict__ v, const float* __restrict__ beta, const float* state_in,
            float* __restrict__ out, float* state_out, int64_t T, int h_qk, int h_v)
{
    constexpr int RPL = D / 16;                     // state rows per lane
    constexpr int NCB = D / 16;                     // 16-column blocks per head
    constexpr int ROWB = SCAN_ST * D * 4;           // bytes of qhat (or khat) rows per stage
    constexpr int NRL = 2 * ROWB / 1024;            // 1 KB row loads per stage (2 .. 16)
    constexpr int NRW = NRL < 4 ? 1 : NRL / 4;      // of them per wave (the excess: none)
    constexpr int VB = SCAN_ST * 16 * (int)sizeof(TIn);  // bytes of value channels per stage
    static_assert(VB <= 1024, "one load covers a stage's value channels");
    constexpr int NDMA = NRW + 1;                   // loads per wave per stage
    constexpr int ES = (int)sizeof(TIn);

    __shared__ __align__(16) float s_rows[SCAN_NSL][2][SCAN_ST * D];  // [slot][qhat, khat]
    __shared__ __align__(16) float s_sc[SCAN_NSL][3][64];             // alpha, beta, qk
    __shared__ __align__(16) char s_v[SCAN_NSL][1024];                // value channels
    __shared__ __align__(16) char s_spare[1024];                      // target of unused loads

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
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane & 15;
    const int cl = wave * 4 + (lane >> 4);  // this lane's channel within the block
    const int j = cb * 16 + cl;             // ... and within the head
    const int row0 = sub * RPL;             // first state row of this lane

    float m[RPL];
    const int64_t sbase = nh * (int64_t)D * D;
#pragma unroll
    for (int r = 0; r < RPL; ++r)
        m[r] = state_in ? state_in[sbase + (int64_t)(row0 + r) * D + j] : 0.f;

    const int64_t nst = (T + SCAN_ST - 1) / SCAN_ST;
    const int64_t row_qk = (int64_t)h_qk * D * 4;  // bytes between tokens of qhat / khat
    const int64_t row_v = (int64_t)h_v * D;        // elements between tokens of v / out
    auto tok_of = [&](int64_t s) { return seq * T + s * SCAN_ST; };
    auto live_of = [&](int64_t s) { return T - s * SCAN_ST < SCAN_ST ? T - s * SCAN_ST : (int64_t)SCAN_ST; };

    // This wave's loads of stage s into ring slot s % SCAN_NSL. Past the last stage every
    // range is empty, so the loads write zeros there (never read).
    auto stage_loads = [&](int64_t s) {
        const int sl = (int)(s % SCAN_NSL);
        const int64_t live = live_of(s);  // may be <= 0
        const int64_t t0 = tok_of(s);
        const int64_t qk_bytes = (live - 1) * row_qk + D * 4;
#pragma unroll
        for (int i = 0; i < NRW; ++i) {
            const int li = wave * NRW + i;  // 1 KB load index within the stage's rows
            const int half = li * 1024 / ROWB;  // 0: qhat, 1: khat
            const int b = li * 1024 - half * ROWB + 16 * lane;
            const int u = b / (D * 4), within = b - u * (D * 4);
            const float* base = (half == 0 ? qhat : khat) + (t0 * h_qk + hq) * (int64_t)D;
            const auto r = make_rsrc(base, qk_bytes);
            void* dst = li < NRL ? (void*)((char*)&s_rows[sl][half][0] + li * 1024 - half * ROWB) : (void*)s_spare;
            load_to_lds(r, dst, li < NRL ? (int)(u * row_qk + within) : (int)OOR);
        }
        if (wave < 3) {  // alpha, beta, qk: one lane per token
            const float* src = wave == 0 ? alpha + t0 * h_v + h : (wave == 1 ? beta + t0 * h_v + h : qkdot + t0 * h_qk + hq);
            const int64_t stride = wave == 2 ? h_qk : h_v;
            const auto r = make_rsrc(src, live > 0 ? ((live - 1) * stride + 1) * 4 : 0);
            load_to_lds4(r, &s_sc[sl][wave][0], lane < SCAN_ST ? (int)(lane * stride * 4) : (int)OOR);
        } else {  // the value channels: 16 * ES bytes per token, 16 bytes per lane
            constexpr int LPT = ES;  // lanes per token
            const int u = lane / LPT, part = lane - u * LPT;
            const auto r = make_rsrc(v + (t0 * h_v + h) * (int64_t)D + cb * 16,
                                     live > 0 ? ((live - 1) * row_v + 16) * ES : 0);
            load_to_lds(r, &s_v[sl][0], u < SCAN_ST ? (int)((u * row_v) * ES + part * 16) : (int)OOR);
        }
    };
    // A store that counts like one (its offset is out of every range, so it writes nothing):
    // keeps the per-stage count of vector memory operations the same from the first stage.
    const auto r_none = make_rsrc(out, 0);
    auto dummy_store = [&]() { __builtin_amdgcn_raw_buffer_store_b32(0u, r_none, (int)OOR, 0, 0); };
    // Waits until this wave's loads of the stage issued 2 NDMA + 3 operations ago are done,
    // then for the other waves: the stage is in LDS for everyone.
    auto wait_stage = [&]() {
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(2 * NDMA + 3) : "memory");
    };

    stage_loads(0);
    dummy_store();
    stage_loads(1);
    dummy_store();
    stage_loads(2);
    dummy_store();
    wait_stage();

    for (int64_t s = 0; s < nst; ++s) {
        stage_loads(s + 3);
        const int sl = (int)(s % SCAN_NSL);
        const int64_t live = live_of(s);
        float obuf = 0.f;  // lane `sub` keeps the output of the stage's token `sub`
        // Tokens past the sequence (u >= live) read zeros for beta, v and the rows, so with
        // alpha taken as 1 their step leaves the state as it is (c = 0): no branch per token.
#pragma unroll
        for (int u = 0; u < SCAN_ST; ++u) {
            float kx[RPL], qx[RPL];
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                kx[r] = s_rows[sl][1][u * D + row0 + r];
                qx[r] = s_rows[sl][0][u * D + row0 + r];
            }
            const float a_t = u < live ? s_sc[sl][0][u] : 1.0f;
            const float b_t = s_sc[sl][1][u], qk_t = s_sc[sl][2][u];
            float v_t;
            if constexpr (ES == 2)
                v_t = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(&s_v[sl][0])[u * 16 + cl]);
            else
                v_t = reinterpret_cast<const float*>(&s_v[sl][0])[u * 16 + cl];
            float sk0 = 0.f, sk1 = 0.f, sq0 = 0.f, sq1 = 0.f;
#pragma unroll
            for (int r = 0; r < RPL; r += 2) {
                sk0 += kx[r] * m[r];
                sq0 += qx[r] * m[r];
                if (r + 1 < RPL) {
                    sk1 += kx[r + 1] * m[r + 1];
                    sq1 += qx[r + 1] * m[r + 1];
                }
            }
            const float sk = row16_sum(sk0 + sk1);
            const float sq = row16_sum(sq0 + sq1);
            const float c = b_t * (v_t - a_t * sk);
            const float o = a_t * sq + c * qk_t;
#pragma unroll
            for (int r = 0; r < RPL; ++r) m[r] = a_t * m[r] + c * kx[r];
            obuf = (sub == u) ? o : obuf;
        }
        {
            const auto r_o = make_rsrc(out + (tok_of(s) * h_v + h) * (int64_t)D,
                                       ((live - 1) * row_v + D) * 4);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(obuf), r_o,
                                                  sub < live ? (int)((sub * row_v + j) * 4) : (int)OOR, 0, 0);
        }
        wait_stage();
    }

#pragma unroll
    for (int r = 0; r < RPL; ++r) state_out[sbase + (int64_t)(row0 + r) * D + j] = m[r];
}

struct ScanWs {
    size_t qhat, khat, qk, alpha, total;
};

ScanWs scan_ws_layout(int64_t n, int64_t t, int32_t h_qk, int32_t h_v, int32_t d)
{
    const size_t rows = (size_t)n * (size_t)t * (size_t)h_qk;
    ScanWs w;
    w.qhat = 0;
    w.khat = align256(rows * d * sizeof(float));
    w.qk = w.khat + align256(rows * d * sizeof(float));
    w.alpha = w.qk + align256(rows * sizeof(float));
    w.total = w.alpha + align256((size_t)n * (size_t)t * (size_t)h_v * sizeof(float));
    return w;
}

template <int D, typename TIn>
hipError_t launch_normalise(const Call& c, const ScanWs& w)
{
    char* ws = static_cast<char*>(c.ws);
    const int64_t rows = c.n * c.t * c.h_qk;
    hipLaunchKernelGGL((qk_normalise_kernel<D, TIn>), dim3((unsigned)((rows + 15) / 16)), dim3(256),
                       0, c.stream, static_cast<const TIn*>(c.q), static_cast<const TIn*>(c.k), c.g,
                       rows, c.h_qk, c.h_v, c.eps, reinterpret_cast<float*>(ws + w.qhat),
                       reinterpret_cast<float*>(ws + w.khat), reinterpret_cast<float*>(ws + w.qk),
                       reinterpret_cast<float*>(ws + w.alpha));
    return hipGetLastError();
}

template <int D, typename TIn>
hipError_t launch_scan_t(const Call& c)
{
    const ScanWs w = scan_ws_layout(c.n, c.t, c.h_qk, c.h_v, D);
    const char* ws = static_cast<const char*>(c.ws);
    hipError_t e = launch_normalise<D, TIn>(c, w);
    if (e != hipSuccess) return e;
    const int64_t blocks = c.n * c.h_v * (D / 16);
    hipLaunchKernelGGL((scan_kernel<D, TIn>), dim3((unsigned)blocks), dim3(256), 0, c.stream,
                       reinterpret_cast<const float*>(ws + w.qhat), reinterpret_cast<const float*>(ws + w.khat),
                       reinterpret_cast<const float*>(ws + w.qk), reinterpret_cast<const float*>(ws + w.alpha),
                       static_cast<const TIn*>(c.v), c.beta, c.state_in, c.out, c.state_out, c.t,
                       c.h_qk, c.h_v);
    return hipGetLastError();
}

// The ablation of state residency: the same normalisation and scan kernels, but the scan is
// launched once per block of block_t tokens of each sequence, so the state leaves the chip
// after every block (written to state_out, read back by the next block's launch).
template <int D, typename TIn>
hipError_t launch_scan_blockwise_t(const Call& c, int64_t block_t)
{
    const ScanWs w = scan_ws_layout(c.n, c.t, c.h_qk, c.h_v, D);
    const char* ws = static_cast<const char*>(c.ws);
    const float* qhat = reinterpret_cast<const float*>(ws + w.qhat);
    const float* khat = reinterpret_cast<const float*>(ws + w.khat);
    const float* qk = reinterpret_cast<const float*>(ws + w.qk);
    const float* alpha = reinterpret_cast<const float*>(ws + w.alpha);
    hipError_t e = launch_normalise<D, TIn>(c, w);
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
                               qk + tok * c.h_qk, alpha + tok * c.h_v, v + tok * c.h_v * D,
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
    return scan_ws_layout(n, t, h_qk, h_v, d).total;
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
