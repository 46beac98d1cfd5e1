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
// One kernel does all of it: the token inputs are staged through LDS well ahead of use, and
// the q/k normalisation and alpha = exp(g) are formed there one stage ahead, so the scan
// needs no workspace.
#include <type_traits>

#include "gdn_internal.hpp"

namespace gdn {
namespace {


// ------------------------------------------------------------------ the scan
// The inputs reach LDS by loads that write it directly, in stages of SCAN_ST tokens, three
// stages ahead of use, into a ring of SCAN_NSL stages: the raw q and k rows of the QK head,
// g, beta and the workgroup's 16 value channels. The loads of a stage are spread evenly over
// the four waves, and each wave waits for its own with an exact count, since per stage it
// issues the same number of vector memory operations (its share of the loads, and one
// store of the stage's outputs). One stage ahead of its use, the four waves normalise a
// stage's rows (qhat = q / sqrt(sum q^2 + eps), khat likewise, qk = qhat . khat, each token
// by one 16-lane row) and form alpha = exp(g), into a second ring of two stages.
constexpr int SCAN_ST = 16;  // tokens per stage
constexpr int SCAN_NSL = 4;  // stages in the ring of raw inputs
constexpr int SCAN_NNS = 2;  // stages in the ring of normalised rows

template <int D, typename TIn>
__global__ void __launch_bounds__(256)
scan_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
            const float* __restrict__ g, const float* __restrict__ beta, const float* state_in,
            float* __restrict__ out, float* state_out, int64_t T, int h_qk, int h_v, float eps)
{
    constexpr int RPL = D / 16;                      // state rows per lane
    constexpr int NCB = D / 16;                      // 16-column blocks per head
    constexpr int ES = (int)sizeof(TIn);
    constexpr int RAWB = SCAN_ST * D * ES;           // bytes of q (or k) rows per stage
    constexpr int RAWP = RAWB < 1024 ? 1024 : RAWB;  // ... padded to whole 1 KB loads
    constexpr int NPB = RAWP / 1024;                 // 1 KB loads per block (q or k)
    constexpr int NRL = 2 * NPB;                     // row loads per stage
    constexpr int NRW = (NRL + 3) / 4;               // of them per wave (the excess: none)
    static_assert(SCAN_ST * 16 * ES <= 1024, "one load covers a stage's value channels");
    constexpr int NDMA = NRW + 1;                    // loads per wave per stage

    __shared__ __align__(16) char s_raw[SCAN_NSL][2][RAWP];      // [slot][q, k] rows
    __shared__ __align__(16) float s_gb[SCAN_NSL][2][64];        // [slot][g, beta]
    __shared__ __align__(16) char s_v[SCAN_NSL][1024];           // value channels
    __shared__ __align__(16) float s_nrm[SCAN_NNS][2][SCAN_ST * D];  // [slot][qhat, khat]
    __shared__ __align__(16) float s_aq[SCAN_NNS][2][SCAN_ST];   // [slot][alpha, qk]
    __shared__ __align__(16) char s_spare[1024];                 // target of unused loads

    // Workgroups that share a QK head's rows (its V heads' column blocks, which are
    // consecutive in `lin`) run on one XCD (blockIdx % 8 picks the XCD), so those rows are
    // fetched into one L2 rather than into all eight.
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
    const int64_t row_qk = (int64_t)h_qk * D * ES;  // bytes between tokens of q / k
    const int64_t row_v = (int64_t)h_v * D;         // elements between tokens of v / out
    auto tok_of = [&](int64_t s) { return seq * T + s * SCAN_ST; };
    auto live_of = [&](int64_t s) { return T - s * SCAN_ST < SCAN_ST ? T - s * SCAN_ST : (int64_t)SCAN_ST; };

    // This wave's loads of stage s into raw slot s % SCAN_NSL. Past the last stage every
    // range is empty, so the loads write zeros there (never read).
    auto stage_loads = [&](int64_t s) {
        const int sl = (int)(s % SCAN_NSL);
        const int64_t live = live_of(s);  // may be <= 0
        const int64_t t0 = tok_of(s);
        const int64_t qk_bytes = (live - 1) * row_qk + D * ES;
#pragma unroll
        for (int i = 0; i < NRW; ++i) {
            const int li = wave * NRW + i;  // 1 KB load index within the stage's rows
            const int which = li / NPB;     // 0: q, 1: k
            const int b = (li - which * NPB) * 1024 + 16 * lane;
            const int u = b / (D * ES), within = b - u * (D * ES);
            const auto r = make_rsrc((which == 0 ? q : k) + (t0 * h_qk + hq) * (int64_t)D, qk_bytes);
            void* dst = li < NRL ? (void*)(&s_raw[sl][which & 1][(li - which * NPB) * 1024]) : (void*)s_spare;
            load_to_lds(r, dst, li < NRL && u < SCAN_ST ? (int)(u * row_qk + within) : (int)OOR);
        }
        if (wave < 2) {  // g, beta: one lane per token
            const float* src = (wave == 0 ? g : beta) + t0 * h_v + h;
            const auto r = make_rsrc(src, live > 0 ? ((live - 1) * h_v + 1) * 4 : 0);
            load_to_lds4(r, &s_gb[sl][wave][0], lane < SCAN_ST ? (int)(lane * h_v * 4) : (int)OOR);
        } else if (wave == 2) {  // the value channels: 16 * ES bytes per token, 16 per lane
            constexpr int LPT = ES;  // lanes per token
            const int u = lane / LPT, part = lane - u * LPT;
            const auto r = make_rsrc(v + (t0 * h_v + h) * (int64_t)D + cb * 16,
                                     live > 0 ? ((live - 1) * row_v + 16) * ES : 0);
            load_to_lds(r, &s_v[sl][0], u < SCAN_ST ? (int)((u * row_v) * ES + part * 16) : (int)OOR);
        } else {  // nothing to load: an empty load, so every wave counts alike
            load_to_lds4(make_rsrc(g, 0), s_spare, (int)OOR);
        }
    };
    // Normalise the rows of stage s (raw slot s % SCAN_NSL) into slot s % SCAN_NNS: token
    // 4 wave + lane / 16, elements row0 .. row0 + RPL - 1 of it in each lane.
    auto normalise = [&](int64_t s) {
        const int rs = (int)(s % SCAN_NSL), ns = (int)(s % SCAN_NNS);
        const int u = 4 * wave + (lane >> 4);
        float qv[RPL], kv[RPL];
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            if constexpr (ES == 2) {
                qv[r] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(&s_raw[rs][0][0])[u * D + row0 + r]);
                kv[r] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(&s_raw[rs][1][0])[u * D + row0 + r]);
            } else {
                qv[r] = reinterpret_cast<const float*>(&s_raw[rs][0][0])[u * D + row0 + r];
                kv[r] = reinterpret_cast<const float*>(&s_raw[rs][1][0])[u * D + row0 + r];
            }
        }
        float qq = 0.f, kk = 0.f, qk = 0.f;
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            qq += qv[r] * qv[r];
            kk += kv[r] * kv[r];
            qk += qv[r] * kv[r];
        }
        qq = row16_sum(qq);
        kk = row16_sum(kk);
        qk = row16_sum(qk);
        const float rq = 1.0f / sqrtf(qq + eps), rk = 1.0f / sqrtf(kk + eps);
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            s_nrm[ns][0][u * D + row0 + r] = qv[r] * rq;
            s_nrm[ns][1][u * D + row0 + r] = kv[r] * rk;
        }
        // every lane of the token's row writes the same two values (no branch)
        s_aq[ns][0][u] = expf(s_gb[rs][0][u]);
        s_aq[ns][1][u] = qk * rq * rk;
    };
    // A store that counts like one (its offset is out of every range, so it writes nothing):
    // keeps the per-stage count of vector memory operations the same from the first stage.
    const auto r_none = make_rsrc(out, 0);
    auto dummy_store = [&]() { __builtin_amdgcn_raw_buffer_store_b32(0u, r_none, (int)OOR, 0, 0); };
    // Waits until this wave's loads issued NDMA + 2 operations ago are done, then for the
    // other waves: those loads' stage is in LDS for everyone.
    auto wait_loads = [&]() {
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(NDMA + 2) : "memory");
    };
    auto barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

    // The tokens of stage s (normalised slot s % SCAN_NNS, raw slot s % SCAN_NSL for beta
    // and v); returns the output this lane keeps (token `sub` of the stage). Full stages
    // run without a branch, with the next stage's normalisation (into the other slot) in
    // their middle, where its independent work fills the gaps of the token chain; the last
    // stage, which may be partial, stops after its `live` tokens.
    auto run_stage = [&](auto partial_c, int64_t s, int64_t live) {
        constexpr bool PARTIAL = decltype(partial_c)::value;
        const int rs = (int)(s % SCAN_NSL), ns = (int)(s % SCAN_NNS);
        float obuf = 0.f;
        auto token = [&](int u) {
            float kx[RPL], qx[RPL];
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                kx[r] = s_nrm[ns][1][u * D + row0 + r];
                qx[r] = s_nrm[ns][0][u * D + row0 + r];
            }
            const float a_t = s_aq[ns][0][u], qk_t = s_aq[ns][1][u], b_t = s_gb[rs][1][u];
            float v_t;
            if constexpr (ES == 2)
                v_t = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(&s_v[rs][0])[u * 16 + cl]);
            else
                v_t = reinterpret_cast<const float*>(&s_v[rs][0])[u * 16 + cl];
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
        };
#pragma unroll
        for (int u = 0; u < SCAN_ST; ++u) {
            if (!PARTIAL && u == SCAN_ST / 2) normalise(s + 1);
            if (!PARTIAL || u < live) token(u);  // wave-uniform
        }
        return obuf;
    };

    stage_loads(0);
    dummy_store();
    stage_loads(1);
    dummy_store();
    stage_loads(2);
    dummy_store();
    wait_loads();  // stages 0 and 1 are in LDS
    normalise(0);
    barrier();

    for (int64_t s = 0; s < nst; ++s) {
        stage_loads(s + 3);
        const int64_t live = live_of(s);
        // every stage but the last normalises the next one; the last may be partial
        const float obuf = s + 1 < nst ? run_stage(std::false_type{}, s, live)
                                       : run_stage(std::true_type{}, s, live);
        {
            const auto r_o = make_rsrc(out + (tok_of(s) * h_v + h) * (int64_t)D,
                                       ((live - 1) * row_v + D) * 4);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(obuf), r_o,
                                                  sub < live ? (int)((sub * row_v + j) * 4) : (int)OOR, 0, 0);
        }
        wait_loads();  // stage s + 2 is in LDS
    }

#pragma unroll
    for (int r = 0; r < RPL; ++r) state_out[sbase + (int64_t)(row0 + r) * D + j] = m[r];
}

template <int D, typename TIn>
hipError_t launch_scan_t(const Call& c)
{
    const int64_t blocks = c.n * c.h_v * (D / 16);
    hipLaunchKernelGGL((scan_kernel<D, TIn>), dim3((unsigned)blocks), dim3(256), 0, c.stream,
                       static_cast<const TIn*>(c.q), static_cast<const TIn*>(c.k),
                       static_cast<const TIn*>(c.v), c.g, c.beta, c.state_in, c.out, c.state_out,
                       c.t, c.h_qk, c.h_v, c.eps);
    return hipGetLastError();
}

// The ablation of state residency: the same scan kernel, launched once per block of
// block_t tokens of each sequence, so the state leaves the chip after every block (written
// to state_out, read back by the next block's launch).
template <int D, typename TIn>
hipError_t launch_scan_blockwise_t(const Call& c, int64_t block_t)
{
    const TIn* q = static_cast<const TIn*>(c.q);
    const TIn* k = static_cast<const TIn*>(c.k);
    const TIn* v = static_cast<const TIn*>(c.v);
    const int64_t state_elems = (int64_t)c.h_v * D * D;
    hipError_t e = hipSuccess;
    for (int64_t s = 0; s < c.n && e == hipSuccess; ++s) {
        for (int64_t t0 = 0; t0 < c.t && e == hipSuccess; t0 += block_t) {
            const int64_t len = c.t - t0 < block_t ? c.t - t0 : block_t;
            const int64_t tok = s * c.t + t0;
            const float* si = t0 == 0 ? (c.state_in ? c.state_in + s * state_elems : nullptr)
                                      : c.state_out + s * state_elems;
            hipLaunchKernelGGL((scan_kernel<D, TIn>), dim3((unsigned)(c.h_v * (D / 16))), dim3(256), 0,
                               c.stream, q + tok * c.h_qk * D, k + tok * c.h_qk * D,
                               v + tok * c.h_v * D, c.g + tok * c.h_v, c.beta + tok * c.h_v, si,
                               c.out + tok * c.h_v * D, c.state_out + s * state_elems, len, c.h_qk,
                               c.h_v, c.eps);
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
    (void)n, (void)t, (void)h_qk, (void)h_v, (void)d;
    return 0;  // the direct scan keeps everything it needs in LDS and registers
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
