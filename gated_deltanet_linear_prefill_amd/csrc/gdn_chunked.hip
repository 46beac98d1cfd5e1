// gdn_chunked.hip -- chunked prefill of the Gated DeltaNet recurrence.
//
// "Optimizing on-device inference for Apple Silicon", section "Qwen creates three distinct
// workload shapes": prefill may re-block the token updates into chunks, which exposes
// matrix work and parallelism over tokens, and computes the same result as the direct
// scan. On MI355X the matrix work goes to bf16 MFMA with fp32 accumulation.
//
// Algebra (per V head, M = S^T of shape d_k x d_v, one chunk of C tokens, M0 the state
// entering it, khat/qhat the L2-normalised keys/queries, gamma_r = g_1 + ... + g_r and
// Gamma_r = exp(gamma_r)). Every value channel j obeys m_r = alpha_r m_{r-1} + khat_r u_r
// with u_r = beta_r (v_r - alpha_r khat_r . m_{r-1}); unrolling m_{r-1} turns the C
// updates into one unit lower triangular system (the UT transform of the delta rule):
//   (I + A) U = diag(beta) V - diag(beta Gamma) Khat M0,
//   A[r][s] = beta_r exp(gamma_r - gamma_s) khat_r . khat_s        (s < r)
// so with T = (I + A)^-1 (WY form):
//   U   = T X,                      X = diag(beta) V - diag(beta Gamma r_k) (K M0)
//   O   = diag(Gamma r_q) (Q M0) + Ptil U,
//         Ptil[r][s] = exp(gamma_r - gamma_s) r_q,r r_k,s q_r . k_s  (s <= r)
//   M_C = Gamma_C M0 + K^T diag(r_k exp(gamma_C - gamma)) U
// where K, Q are the raw inputs and r_k, r_q the inverse norms: the normalisation is kept
// as diagonal scalings so the bf16 inputs enter the MFMAs exactly. Decays only appear as
// exp(gamma_r - gamma_s) with s <= r, never as 1/Gamma, so nothing overflows.
//
// Two kernels:
//  * chunk_prep_kernel (one workgroup per sequence, chunk and QK head; fully parallel):
//    inverse norms, gate prefix sums, K K^T and Q K^T on MFMA, A, T = (I + A)^-1 by
//    blocked forward substitution in LDS (16x16 diagonal blocks by substitution, the
//    off-diagonal blocks with fp32 MFMA), and writes to the workspace T and Ptil as
//    hi/lo bf16 pairs already in MFMA A-operand order, K^T tiles, and per-token scalars.
//  * chunk_scan_kernel (one workgroup per sequence, V head and 16 value channels;
//    sequential over chunks): the state block stays in MFMA accumulators for the whole
//    call; per chunk K M0 and Q M0, X, U = T X, O and the state update run on MFMA.
//
// Decay factors exp(gamma_r - gamma_s) <= 1 inside the C x C matrices use the hardware
// exponential (__expf); its relative error, a few 1e-6 at these arguments, is far below the
// split-bf16 operand precision.
//
// Precision: an MFMA operand that is not an exact bf16 input (the state, X, U, T, Ptil) is
// split into hi = bf16(x) and lo = bf16(x - hi) and multiplied as hi*hi + hi*lo + lo*hi
// (or hi + lo against an exact operand), which keeps about 16 significant bits per
// operand and fp32 accumulation; rounding them to one bf16 would not meet the accuracy
// the recurrence needs (the page's "Keep the recurrent state on-chip" section keeps the
// state and gate in 32-bit floats for the same reason).
#include <type_traits>

#include "gdn_internal.hpp"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma_bf16(bf16x8 a, bf16x8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma_f32(float a, float b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo)
{
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

// Wait for this wave's LDS traffic and keep the compiler from moving memory accesses
// across the point (used between a wave's own LDS write and read-back).
__device__ __forceinline__ void lds_fence()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// MFMA 16x16x32 operand conventions used throughout (lane l, lr = l & 15, lg = l >> 4):
//   A fragment (16 rows x 32 k): row lr, k = 8 lg + 0..7
//   B fragment (32 k x 16 cols): col lr, k = 8 lg + 0..7
//   accumulator (16 x 16 fp32):  rows 4 lg + 0..3, col lr
// Only the row/column roles matter: A and B enumerate k the same way, so the contraction
// is the same whatever order the hardware pairs the eight elements in.

template <int D, int C, bool F32IN>
struct Geo {
    static constexpr int DP = D < 32 ? 32 : D;  // contraction over d, padded to k = 32
    static constexpr int CP = C < 32 ? 32 : C;  // contraction over chunk tokens, padded
    static constexpr int RT = C / 16;           // 16-token row tiles of a chunk
    static constexpr int KTC = CP / 32;         // k tiles over chunk tokens
    static constexpr int KTD = DP / 32;         // k tiles over d
    static constexpr int MT = D / 16;           // 16-row tiles of the state (d_k)
    static constexpr int NS = F32IN ? 2 : 1;    // bf16 pieces per q/k element
    static constexpr size_t KT_BYTES = (size_t)MT * KTC * NS * 1024;  // per (chunk, QK head)
    static constexpr size_t TP_BYTES = (size_t)RT * KTC * 2 * 1024;   // per (chunk, V head)
    static constexpr size_t SC_BYTES = (size_t)C * 16;                // per (chunk, V head)
};

// Workspace regions; every region starts 256-byte aligned.
struct ChunkWs {
    int64_t nch;                    // chunks per sequence
    size_t kt, t, p, sc, gc, total; // byte offsets
    size_t kt_bytes, tp_bytes, sc_bytes;
};

size_t align256(size_t x)
{
    return (x + 255) & ~size_t(255);
}

ChunkWs chunk_ws(int64_t n, int64_t t, int32_t h_qk, int32_t h_v, int32_t d, int chunk,
                 bool f32in)
{
    const int dp = d < 32 ? 32 : d, cp = chunk < 32 ? 32 : chunk;
    (void)dp;
    ChunkWs w;
    w.nch = (t + chunk - 1) / chunk;
    w.kt_bytes = (size_t)(d / 16) * (cp / 32) * (f32in ? 2 : 1) * 1024;
    w.tp_bytes = (size_t)(chunk / 16) * (cp / 32) * 2 * 1024;
    w.sc_bytes = (size_t)chunk * 16;
    const size_t nq = (size_t)n * w.nch * h_qk, nv = (size_t)n * w.nch * h_v;
    w.kt = 0;
    w.t = w.kt + align256(nq * w.kt_bytes);
    w.p = w.t + align256(nv * w.tp_bytes);
    w.sc = w.p + align256(nv * w.tp_bytes);
    w.gc = w.sc + align256(nv * w.sc_bytes);
    w.total = w.gc + align256(nv * sizeof(float));
    return w;
}

// Eight consecutive q/k elements as bf16 fragment pieces: the exact value for bf16
// input; hi and lo for fp32 input; zero when !ok. `p` must point to readable memory even
// when !ok: the load is unconditional and the mask is a select, so no branch (and no
// early wait on outstanding loads) is tied to the lane predicate.
template <typename TIn>
__device__ __forceinline__ void load_frag(const TIn* p, bool ok, bf16x8* piece)
{
    if constexpr (std::is_same<TIn, float>::value) {
        const float4 a = reinterpret_cast<const float4*>(p)[0];
        const float4 b = reinterpret_cast<const float4*>(p)[1];
        const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        bf16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            __bf16 h, l;
            split_bf16(ok ? x[e] : 0.f, h, l);
            hi[e] = h;
            lo[e] = l;
        }
        piece[0] = hi;
        piece[1] = lo;
    } else {
        const bf16x8 val = *reinterpret_cast<const bf16x8*>(p);
        bf16x8 zero;
#pragma unroll
        for (int e = 0; e < 8; ++e) zero[e] = (__bf16)0.f;
        piece[0] = ok ? val : zero;
    }
}

// Raw fragment storage for the scan kernel's prefetch registers: the loaded bits are kept
// as they arrive and turned into MFMA pieces at use, so issuing the next chunk's loads
// never has to wait for them.
typedef float floatx8 __attribute__((ext_vector_type(8)));
template <typename TIn>
struct RawFrag;
template <>
struct RawFrag<uint16_t> {
    using type = bf16x8;
};
template <>
struct RawFrag<float> {
    using type = floatx8;
};

template <typename TIn>
__device__ __forceinline__ typename RawFrag<TIn>::type load_raw_frag(const TIn* p)
{
    return *reinterpret_cast<const typename RawFrag<TIn>::type*>(p);
}

__device__ __forceinline__ void to_pieces(const bf16x8& raw, bf16x8* piece)
{
    piece[0] = raw;
}

__device__ __forceinline__ void to_pieces(const floatx8& raw, bf16x8* piece)
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        __bf16 h, l;
        split_bf16(raw[e], h, l);
        piece[0][e] = h;
        piece[1][e] = l;
    }
}

__device__ __forceinline__ float raw_to_f32(uint16_t x)
{
    return bf16_bits_to_f32(x);
}

__device__ __forceinline__ float raw_to_f32(float x)
{
    return x;
}

// Buffer resources: a base address and byte range in scalar registers, re-based once per
// chunk with scalar adds, while each lane keeps one fixed byte offset. Lanes whose offset
// falls outside the range read zero (and their stores are dropped), which handles the rows
// past the end of a sequence without per-lane branches. The 0x00020000 word is the raw
// (untyped, unswizzled) descriptor format of the gfx9 family.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes)
{
    const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

__device__ __forceinline__ bf16x8 buf_bf16x8(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ u32x4 buf_u32x4(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ floatx4 buf_floatx4(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <typename TIn>
__device__ __forceinline__ TIn buf_elem(__amdgpu_buffer_rsrc_t r, int off);

template <>
__device__ __forceinline__ uint16_t buf_elem<uint16_t>(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

template <>
__device__ __forceinline__ float buf_elem<float>(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

template <typename TIn>
__device__ __forceinline__ typename RawFrag<TIn>::type buf_raw_frag(__amdgpu_buffer_rsrc_t r, int off);

template <>
__device__ __forceinline__ bf16x8 buf_raw_frag<uint16_t>(__amdgpu_buffer_rsrc_t r, int off)
{
    return buf_bf16x8(r, off);
}

template <>
__device__ __forceinline__ floatx8 buf_raw_frag<float>(__amdgpu_buffer_rsrc_t r, int off)
{
    const floatx4 a = buf_floatx4(r, off), b = buf_floatx4(r, off + 16);
    return floatx8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// acc += A * B with A given as NA bf16 pieces and B as NB pieces, skipping lo*lo.
template <int NA, int NB>
__device__ __forceinline__ floatx4 mfma_split(const bf16x8* a, const bf16x8* b, floatx4 acc)
{
    acc = mfma_bf16(a[0], b[0], acc);
    if constexpr (NB > 1) acc = mfma_bf16(a[0], b[1], acc);
    if constexpr (NA > 1) acc = mfma_bf16(a[1], b[0], acc);
    return acc;
}

// The same product with each split pass in its own accumulator (acc[0..NA+NB-2]), so the
// passes do not wait on each other; the caller sums the accumulators at the end.
template <int NA, int NB>
__device__ __forceinline__ void mfma_split_acc(const bf16x8* a, const bf16x8* b, floatx4* acc)
{
    acc[0] = mfma_bf16(a[0], b[0], acc[0]);
    if constexpr (NB > 1) acc[1] = mfma_bf16(a[0], b[1], acc[1]);
    if constexpr (NA > 1) acc[NB] = mfma_bf16(a[1], b[0], acc[NB]);
}

// Index of the t-th lower-triangular 16x16 tile (row tile >= column tile).
__device__ __forceinline__ void tri_tile(int t, int& rt, int& ct)
{
    rt = 0;
    while ((rt + 1) * (rt + 2) / 2 <= t) ++rt;
    ct = t - rt * (rt + 1) / 2;
}

// =============================================================================== prep
template <int D, int C, typename TIn>
__global__ void __launch_bounds__(256)
chunk_prep_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const float* __restrict__ g,
                  const float* __restrict__ beta, char* __restrict__ ws, ChunkWs L, int64_t T,
                  int h_qk, int h_v, float eps)
{
    constexpr bool F32IN = std::is_same<TIn, float>::value;
    using G = Geo<D, C, F32IN>;
    constexpr int DP = G::DP, RT = G::RT, KTC = G::KTC, KTD = G::KTD, MT = G::MT, NS = G::NS;
    constexpr int NB = C / 16;    // 16x16 diagonal blocks of T
    constexpr int KS = DP + 8;    // LDS row stride of the K chunk (bf16)
    constexpr int CS = C + 4;     // LDS row stride of the C x C fp32 matrices
    constexpr size_t K_LDS = (size_t)NS * C * KS * 2;
    constexpr size_t AT_LDS = (size_t)2 * C * CS * 4;
    constexpr size_t U_LDS = K_LDS > AT_LDS ? K_LDS : AT_LDS;

    // The K chunk (phase 0) and the A / T matrices (later phases) share one buffer.
    __shared__ __align__(16) char s_buf[U_LDS];
    __shared__ float s_rk[C], s_rq[C], s_gam[C], s_beta[C];
    __shared__ float s_x[4][16][17];  // per-wave 16x16 scratch
    auto s_k = [&](int part, int r, int f) -> __bf16& {
        return reinterpret_cast<__bf16*>(s_buf)[((size_t)part * C + r) * KS + f];
    };
    float(*s_a)[CS] = reinterpret_cast<float(*)[CS]>(s_buf);
    float(*s_t)[CS] = reinterpret_cast<float(*)[CS]>(s_buf + (size_t)C * CS * 4);

    const int64_t nch = L.nch;
    const int hq = (int)(blockIdx.x % h_qk);
    const int64_t sc_idx = blockIdx.x / h_qk;
    const int64_t c = sc_idx % nch, seq = sc_idx / nch;
    const int64_t c0 = c * C;
    const int Cr = (int)((T - c0) < C ? (T - c0) : C);
    const int tid = threadIdx.x, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
    const int grp = h_v / h_qk;
    const int64_t tok0 = seq * T + c0;  // flattened token index of the chunk's first token

    // ---- phase 0: inverse norms of q and k rows; the K chunk into LDS as bf16 pieces
    {
        constexpr int EPL = D / 16;  // elements per lane, 16 lanes per row
        const int sub = tid & 15;
        for (int r0 = 0; r0 < C; r0 += 16) {
            const int r = r0 + (tid >> 4);
            const bool ok = r < Cr;
            const int64_t off = ((tok0 + (ok ? r : 0)) * h_qk + hq) * (int64_t)D + sub * EPL;
            float qv[EPL], kv[EPL];
            load_n<EPL>(q + off, qv);
            load_n<EPL>(k + off, kv);
            float qq = 0.f, kk = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                qq += qv[e] * qv[e];
                kk += kv[e] * kv[e];
            }
            qq = row16_sum(qq);
            kk = row16_sum(kk);
            if (sub == 0) {
                s_rq[r] = ok ? 1.0f / sqrtf(qq + eps) : 0.f;
                s_rk[r] = ok ? 1.0f / sqrtf(kk + eps) : 0.f;
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                __bf16 hi, lo;
                split_bf16(ok ? kv[e] : 0.f, hi, lo);
                s_k(0, r, sub * EPL + e) = hi;
                if constexpr (NS > 1) s_k(1, r, sub * EPL + e) = lo;
            }
            if constexpr (D < DP) {  // zero the padded features
#pragma unroll
                for (int e = 0; e < (DP - D) / 16; ++e)
                    for (int part = 0; part < NS; ++part)
                        s_k(part, r, D + sub * ((DP - D) / 16) + e) = (__bf16)0.f;
            }
        }
    }
    __syncthreads();

    // ---- K^T tiles (A operand of K^T W in the scan kernel): tile (mt, kt, part) holds
    //      K[token 32 kt + 8 lg + e][feature 16 mt + lr]
    {
        char* kt_base = ws + L.kt + (size_t)((seq * nch + c) * h_qk + hq) * G::KT_BYTES;
        constexpr int NTILE = MT * KTC * NS;
        for (int ti = w; ti < NTILE; ti += 4) {
            const int part = ti % NS, kt = (ti / NS) % KTC, mt = ti / (NS * KTC);
            const int f = 16 * mt + lr, r0 = 32 * kt + 8 * lg;
            bf16x8 val;
#pragma unroll
            for (int e = 0; e < 8; ++e) val[e] = (r0 + e < C) ? s_k(part, r0 + e, f) : (__bf16)0.f;
            *reinterpret_cast<bf16x8*>(kt_base + (size_t)ti * 1024 + l * 16) = val;
        }
    }
    __syncthreads();  // the K buffer becomes A / T below

    // Fragments of the q/k rows of this chunk, straight from the input tensors.
    auto qk_frag = [&](const TIn* base, int row, int kt, bf16x8* piece) {
        const int f = 32 * kt + 8 * lg;
        const bool ok = row < Cr && f < D;
        load_frag<TIn>(base + ((tok0 + (ok ? row : 0)) * h_qk + hq) * (int64_t)D + (ok ? f : 0), ok,
                       piece);
    };

    constexpr int NTL = RT * (RT + 1) / 2;  // lower-triangular 16x16 tiles of a C x C matrix
    for (int gi = 0; gi < grp; ++gi) {
        const int hv = hq * grp + gi;
        const int64_t vh = (seq * nch + c) * h_v + hv;

        // ---- phase 1: gate prefix sums gamma (wave 0), per-token scalars
        if (w == 0) {
            constexpr int E = (C + 63) / 64;
            float gv[E], bv[E];
            float run = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int i = l * E + e;
                const bool ok = i < Cr;
                const int64_t gi_off = (tok0 + (ok ? i : 0)) * h_v + hv;
                const float g_in = g[gi_off], b_in = beta[gi_off];
                gv[e] = ok ? g_in : 0.f;
                bv[e] = ok ? b_in : 0.f;
                run += gv[e];
                gv[e] = run;
            }
            float x = run;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (l >= off) x += y;
            }
            const float excl = x - run;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int i = l * E + e;
                if (i < C) {
                    s_gam[i] = gv[e] + excl;
                    s_beta[i] = bv[e];
                }
            }
        }
        __syncthreads();
        {
            const float gam_c = s_gam[C - 1];  // padded tokens add g = 0
            if (tid < C) {
                const int i = tid;
                const float Gi = expf(s_gam[i]);
                float4 o;
                o.x = s_beta[i];                         // beta_r
                o.y = s_beta[i] * Gi * s_rk[i];          // beta_r Gamma_r r_k,r
                o.z = Gi * s_rq[i];                      // Gamma_r r_q,r
                o.w = s_rk[i] * expf(gam_c - s_gam[i]);  // r_k,r exp(gamma_C - gamma_r)
                reinterpret_cast<float4*>(ws + L.sc + (size_t)vh * G::SC_BYTES)[i] = o;
            }
            if (tid == 0) reinterpret_cast<float*>(ws + L.gc)[vh] = expf(gam_c);
        }

        // ---- phase 2: A = strictly lower (beta_r exp(gamma_r - gamma_s) r_k,r r_k,s k_r . k_s)
        for (int ti = w; ti < NTL; ti += 4) {
            int rt, ct;
            tri_tile(ti, rt, ct);
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < KTD; ++kt) {
                bf16x8 a[NS], b[NS];
                qk_frag(k, 16 * rt + lr, kt, a);
                qk_frag(k, 16 * ct + lr, kt, b);
                acc = mfma_split<NS, NS>(a, b, acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + 4 * lg + e, s = 16 * ct + lr;
                float a = 0.f;
                if (s < r) a = s_beta[r] * __expf(s_gam[r] - s_gam[s]) * s_rk[r] * s_rk[s] * acc[e];
                s_a[r][s] = a;
            }
        }
        __syncthreads();

        // ---- phase 3: diagonal 16x16 blocks of T by forward substitution, one lane per
        //      column: T[r][s] = delta_rs - sum_{m<r} A[r][m] T[m][s]
        if (tid < NB * 16) {
            const int b = tid >> 4, s = tid & 15;
            float t[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == s) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) acc -= s_a[16 * b + r][16 * b + m] * t[m];
                t[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) s_t[16 * b + r][16 * b + s] = t[r];
        }
        __syncthreads();

        // ---- phase 4: off-diagonal blocks, block row by block row:
        //      T_ij = -T_ii (sum_{m=j}^{i-1} A_im T_mj)   (fp32 MFMA)
        for (int i = 1; i < NB; ++i) {
            for (int j = w; j < i; j += 4) {
                floatx4 x = {0.f, 0.f, 0.f, 0.f};
                for (int m = j; m < i; ++m) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        x = mfma_f32(s_a[16 * i + lr][16 * m + 4 * kk + lg],
                                     s_t[16 * m + 4 * kk + lg][16 * j + lr], x);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) s_x[w][4 * lg + e][lr] = x[e];
                lds_fence();
                floatx4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    y = mfma_f32(s_t[16 * i + lr][16 * i + 4 * kk + lg], s_x[w][4 * kk + lg][lr], y);
#pragma unroll
                for (int e = 0; e < 4; ++e) s_t[16 * i + 4 * lg + e][16 * j + lr] = -y[e];
                lds_fence();
            }
            __syncthreads();
        }

        // ---- write a lower-triangular C x C matrix as hi/lo MFMA A-operand tiles
        auto write_tiles = [&](float(*src)[CS], char* base) {
            for (int ti = w; ti < RT * KTC; ti += 4) {
                const int rt = ti / KTC, kt = ti % KTC;
                if (32 * kt > 16 * rt + 15) continue;  // above the diagonal: never read
                const int r = 16 * rt + lr, s0 = 32 * kt + 8 * lg;
                bf16x8 hi, lo;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s = s0 + e;
                    const float x = (s <= r && s < C) ? src[r][s] : 0.f;
                    __bf16 h, lw;
                    split_bf16(x, h, lw);
                    hi[e] = h;
                    lo[e] = lw;
                }
                *reinterpret_cast<bf16x8*>(base + (size_t)(2 * ti) * 1024 + l * 16) = hi;
                *reinterpret_cast<bf16x8*>(base + (size_t)(2 * ti + 1) * 1024 + l * 16) = lo;
            }
        };
        write_tiles(s_t, ws + L.t + (size_t)vh * G::TP_BYTES);

        // ---- phase 5: Ptil = lower (exp(gamma_r - gamma_s) r_q,r r_k,s q_r . k_s), into A's space
        for (int ti = w; ti < NTL; ti += 4) {
            int rt, ct;
            tri_tile(ti, rt, ct);
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < KTD; ++kt) {
                bf16x8 a[NS], b[NS];
                qk_frag(q, 16 * rt + lr, kt, a);
                qk_frag(k, 16 * ct + lr, kt, b);
                acc = mfma_split<NS, NS>(a, b, acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + 4 * lg + e, s = 16 * ct + lr;
                float p = 0.f;
                if (s <= r) p = __expf(s_gam[r] - s_gam[s]) * s_rq[r] * s_rk[s] * acc[e];
                s_a[r][s] = p;
            }
        }
        __syncthreads();
        write_tiles(s_a, ws + L.p + (size_t)vh * G::TP_BYTES);
        __syncthreads();
    }
}

// =============================================================================== scan
template <int D, int C, typename TIn>
struct ChunkRegs {
    using G = Geo<D, C, std::is_same<TIn, float>::value>;
    using Raw = typename RawFrag<TIn>::type;
    // bf16 K and Q chunks are staged through LDS with coalesced loads (a 16-lane group reads
    // one contiguous 256-byte row); fp32 inputs (small head dims) load MFMA fragments
    // directly and split them at use.
    static constexpr bool KQ_LDS = !std::is_same<TIn, float>::value;
    static constexpr int RTW = (G::RT + 3) / 4;          // row tiles per wave
    static constexpr int MTW = (G::MT + 3) / 4;          // state row tiles per wave
    static constexpr int NPIECE = C * D / 8;             // 16-byte pieces of a K (or Q) chunk
    static constexpr int KQP = (NPIECE + 255) / 256;     // pieces per thread
    static constexpr int NFRAG = KQ_LDS ? 1 : RTW;
    static constexpr int NKTD = KQ_LDS ? 1 : G::KTD;
    u32x4 kp[KQ_LDS ? KQP : 1], qp[KQ_LDS ? KQP : 1];     // K, Q pieces of the chunk (LDS path)
    Raw ka[NFRAG][NKTD], qa[NFRAG][NKTD];                 // K, Q fragments (direct path)
    TIn vv[RTW][4];                                       // V in accumulator layout, as loaded
    floatx4 scv;                                          // one token's scalars (LDS path)
    floatx4 sc[KQ_LDS ? 1 : RTW][4];                      // per-token scalars (direct path)
    bf16x8 tf[RTW][G::KTC][2], pf[RTW][G::KTC][2];        // T, Ptil (hi, lo)
    bf16x8 kt[KQ_LDS ? 1 : MTW][KQ_LDS ? 1 : G::KTC][G::NS];  // K^T tiles (direct path)
    float gc;                                             // Gamma_C
};

template <int D, int C, typename TIn>
__global__ void __launch_bounds__(256)
chunk_scan_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
                  const char* __restrict__ ws, ChunkWs L, const float* state_in,
                  float* __restrict__ out, float* state_out, int64_t T, int h_qk, int h_v,
                  int64_t nblocks)
{
    constexpr bool F32IN = std::is_same<TIn, float>::value;
    using G = Geo<D, C, F32IN>;
    using R = ChunkRegs<D, C, TIn>;
    constexpr int DP = G::DP, CP = G::CP, RT = G::RT, KTC = G::KTC, KTD = G::KTD, MT = G::MT;
    constexpr int NS = G::NS, RTW = R::RTW, MTW = R::MTW;
    constexpr bool KQ_LDS = R::KQ_LDS;
    constexpr int NCB = D / 16;
    constexpr int MS = DP + 8;  // LDS stride of M^T rows (bf16)
    constexpr int XS = CP + 8;  // LDS stride of X^T, U^T, W^T rows (bf16)
    constexpr int KS = DP + 8;  // LDS stride of K / Q chunk rows (bf16)

    // B operands built in-kernel, stored transposed (value channel major) so that a lane's
    // eight k-consecutive elements are contiguous; and the K / Q chunk (A operands).
    __shared__ __align__(16) __bf16 s_m[2][16][MS];  // state block (hi, lo)
    __shared__ __align__(16) __bf16 s_x[2][16][XS];  // X
    __shared__ __align__(16) __bf16 s_u[2][16][XS];  // U
    __shared__ __align__(16) __bf16 s_w[2][16][XS];  // W = diag(r_k exp(gamma_C - gamma)) U
    // K rows (two buffers by chunk parity: read up to the state update), Q rows (read only
    // before the first barrier) and per-token scalars (two buffers).
    __shared__ __align__(16) __bf16 s_k[2][KQ_LDS ? C : 1][KQ_LDS ? KS : 8];
    __shared__ __align__(16) __bf16 s_q[KQ_LDS ? C : 1][KQ_LDS ? KS : 8];
    __shared__ __align__(16) floatx4 s_sc[2][KQ_LDS ? C : 1];

    // Workgroups that share a QK head run on the same XCD (blockIdx % 8 picks the XCD), so
    // their common K/Q/T/Ptil reads meet in one L2.
    int64_t lin = blockIdx.x;
    if (nblocks % 8 == 0) lin = (int64_t)(blockIdx.x % 8) * (nblocks / 8) + blockIdx.x / 8;
    const int cb = (int)(lin % NCB);
    const int64_t nh = lin / NCB;
    const int64_t seq = nh / h_v;
    const int h = (int)(nh - seq * h_v);
    const int hq = h / (h_v / h_qk);
    const int tid = threadIdx.x, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
    const int64_t nch = L.nch;

    // Zero every LDS operand buffer once: padded k ranges (features >= D, tokens >= C) are
    // never written and must read as zero.
    {
        auto zero = [&](__bf16* z, int n) {
            for (int i = tid; i < n; i += 256) z[i] = (__bf16)0.f;
        };
        zero(&s_m[0][0][0], 2 * 16 * MS);
        zero(&s_x[0][0][0], 2 * 16 * XS);
        zero(&s_u[0][0][0], 2 * 16 * XS);
        zero(&s_w[0][0][0], 2 * 16 * XS);
        if constexpr (KQ_LDS) {
            zero(&s_k[0][0][0], 2 * C * KS);
            zero(&s_q[0][0], C * KS);
        }
    }
    __syncthreads();

    // Four accumulator rows of one column, split, as two 8-byte LDS stores (hi, lo).
    auto put4 = [&](__bf16* hi_row, __bf16* lo_row, floatx4 val) {
        bf16x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            __bf16 hh, ll;
            split_bf16(val[e], hh, ll);
            hi[e] = hh;
            lo[e] = ll;
        }
        *reinterpret_cast<bf16x4*>(hi_row) = hi;
        *reinterpret_cast<bf16x4*>(lo_row) = lo;
    };

    // State block in accumulator layout: tile mt = w + 4 i holds M[16 mt + 4 lg + e][cb 16 + lr].
    floatx4 macc[MTW];
    const int64_t sbase = nh * (int64_t)D * D;
    auto store_m_lds = [&](int i, int mt) {
        put4(&s_m[0][lr][16 * mt + 4 * lg], &s_m[1][lr][16 * mt + 4 * lg], macc[i]);
    };
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
        const int mt = w + 4 * i;
        if (mt < MT) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                macc[i][e] = state_in ? state_in[sbase + (int64_t)(16 * mt + 4 * lg + e) * D + cb * 16 + lr]
                                      : 0.f;
            store_m_lds(i, mt);
        }
    }

    // Byte strides and this lane's fixed byte offsets inside each per-chunk buffer range.
    constexpr int ES = sizeof(TIn);
    const int64_t row_qk = (int64_t)h_qk * D * ES;  // between consecutive tokens of q, k
    const int64_t row_v = (int64_t)h_v * D * ES;    // ... of v
    const int64_t row_o = (int64_t)h_v * D * 4;     // ... of out
    int off_v[RTW][4], off_o[RTW][4];
#pragma unroll
    for (int i = 0; i < RTW; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int rr = 16 * (w + 4 * i) + 4 * lg + e;
            off_v[i][e] = (int)(rr * row_v) + lr * ES;
            off_o[i][e] = (int)(rr * row_o) + lr * 4;
        }

    auto load = [&](R& x, int64_t c) {
        c = c < nch ? c : nch - 1;  // past the end: reload the last chunk (never computed)
        const int64_t c0 = c * C;
        const int64_t tok0 = seq * T + c0;
        const int64_t rows = (T - c0) < C ? (T - c0) : C;  // tokens of this chunk
        const int64_t vh = (seq * nch + c) * h_v + h;
        const auto r_t = make_rsrc(ws + L.t + (size_t)vh * G::TP_BYTES, G::TP_BYTES);
        const auto r_p = make_rsrc(ws + L.p + (size_t)vh * G::TP_BYTES, G::TP_BYTES);
        const auto r_sc = make_rsrc(ws + L.sc + (size_t)vh * G::SC_BYTES, G::SC_BYTES);
        const auto r_kt = make_rsrc(ws + L.kt + (size_t)((seq * nch + c) * h_qk + hq) * G::KT_BYTES,
                                    G::KT_BYTES);
        // q / k rows of QK head hq and the v block of this workgroup; rows past the end
        // fall outside the range and read zero.
        const int64_t kq_bytes = (rows - 1) * row_qk + D * ES;
        const auto r_k = make_rsrc(k + (tok0 * h_qk + hq) * (int64_t)D, kq_bytes);
        const auto r_q = make_rsrc(q + (tok0 * h_qk + hq) * (int64_t)D, kq_bytes);
        const auto r_v = make_rsrc(v + (tok0 * h_v + h) * (int64_t)D + cb * 16, (rows - 1) * row_v + 16 * ES);
        if constexpr (KQ_LDS) {
#pragma unroll
            for (int p = 0; p < R::KQP; ++p) {
                const int pidx = tid + 256 * p;
                const int r = (pidx / (D / 8)) % C, f = (pidx % (D / 8)) * 8;
                const int off = (int)(r * row_qk) + f * ES;
                x.kp[p] = buf_u32x4(r_k, off);
                x.qp[p] = buf_u32x4(r_q, off);
            }
            x.scv = buf_floatx4(r_sc, (tid % C) * 16);
        }
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = w + 4 * i;
            if (rt >= RT) continue;
            if constexpr (!KQ_LDS) {
                // Padded features (f >= D) read zero through an out-of-range offset.
#pragma unroll
                for (int kt = 0; kt < KTD; ++kt) {
                    const int f = 32 * kt + 8 * lg;
                    const int off = f < D ? (int)((16 * rt + lr) * row_qk) + f * ES : 0x7fffffff - 64;
                    x.ka[i][kt] = buf_raw_frag<TIn>(r_k, off);
                    x.qa[i][kt] = buf_raw_frag<TIn>(r_q, off);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x.vv[i][e] = buf_elem<TIn>(r_v, off_v[i][e]);
                if constexpr (!KQ_LDS) x.sc[i][e] = buf_floatx4(r_sc, (16 * rt + 4 * lg + e) * 16);
            }
#pragma unroll
            for (int kt = 0; kt < KTC; ++kt) {
                if (32 * kt > 16 * rt + 15) continue;
                const int o = (rt * KTC + kt) * 2 * 1024 + l * 16;
                x.tf[i][kt][0] = buf_bf16x8(r_t, o);
                x.tf[i][kt][1] = buf_bf16x8(r_t, o + 1024);
                x.pf[i][kt][0] = buf_bf16x8(r_p, o);
                x.pf[i][kt][1] = buf_bf16x8(r_p, o + 1024);
            }
        }
        if constexpr (!KQ_LDS) {
#pragma unroll
            for (int i = 0; i < MTW; ++i) {
                const int mt = w + 4 * i;
                if (mt >= MT) continue;
#pragma unroll
                for (int kt = 0; kt < KTC; ++kt)
#pragma unroll
                    for (int part = 0; part < NS; ++part)
                        x.kt[i][kt][part] = buf_bf16x8(r_kt, ((mt * KTC + kt) * NS + part) * 1024 + l * 16);
            }
        }
        // A vector load (every lane the same word), not a scalar one: scalar loads share the
        // LDS wait counter, and the wait before each barrier would stall on its round trip.
        x.gc = buf_elem<float>(make_rsrc(ws + L.gc + (size_t)vh * 4, 4), 0);
    };

    // K / Q pieces and scalars of a chunk into LDS buffer `b` (rows past the end arrived as
    // zero).
    auto store_kq = [&](const R& x, int b) {
        if constexpr (KQ_LDS) {
#pragma unroll
            for (int p = 0; p < R::KQP; ++p) {
                const int pidx = tid + 256 * p;
                if (R::NPIECE % 256 != 0 && pidx >= R::NPIECE) continue;
                const int r = pidx / (D / 8), f = (pidx % (D / 8)) * 8;
                *reinterpret_cast<u32x4*>(&s_k[b][r][f]) = x.kp[p];
                *reinterpret_cast<u32x4*>(&s_q[r][f]) = x.qp[p];
            }
            if (tid < C) s_sc[b][tid] = x.scv;
        }
    };

    // Outputs of a chunk wait in registers and are stored after the next wait for loads:
    // vector-memory loads and stores share one completion counter, so a store issued just
    // before that wait would stall it for the write round trip.
    floatx4 opend[RTW];
    auto store_out = [&](int64_t c) {
        const int64_t c0 = c * C;
        const int64_t rows = (T - c0) < C ? (T - c0) : C;
        const auto r_o = make_rsrc(out + ((seq * T + c0) * h_v + h) * (int64_t)D + cb * 16,
                                   (rows - 1) * row_o + 64);
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = w + 4 * i;
            if (rt >= RT) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // Element to a scalar first: a bit cast of a vector-element expression picked
                // element 0 for every e in this compiler.
                const float val = opend[i][e];
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), r_o, off_o[i][e], 0, 0);
            }
        }
    };

    // Scalars {beta, beta Gamma r_k, Gamma r_q, r_k exp(gamma_C - gamma)} of accumulator
    // row e of row tile w + 4 i.
    auto scal = [&](const R& x, int b, int i, int e) -> floatx4 {
        if constexpr (KQ_LDS) return s_sc[b][16 * (w + 4 * i) + 4 * lg + e];
        else return x.sc[i][e];
    };

    auto compute = [&](const R& x, int b) {
        // (1) K M0 and Q M0; X = diag(beta) V - diag(beta Gamma r_k) K M0
        floatx4 qm[RTW];
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = w + 4 * i;
            if (rt >= RT) continue;
            // Independent accumulators per k-tile parity and split pass (summed below), so
            // consecutive MFMAs do not wait on each other's results.
            constexpr int NP = NS + 1;  // passes per k tile: M hi, M lo (and K lo)
            floatx4 kacc[2][NP], qacc[2][NP];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int pp = 0; pp < NP; ++pp) kacc[j][pp] = qacc[j][pp] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < KTD; ++kt) {
                bf16x8 mb[2], ka[NS], qa[NS];
                mb[0] = *reinterpret_cast<const bf16x8*>(&s_m[0][lr][32 * kt + 8 * lg]);
                mb[1] = *reinterpret_cast<const bf16x8*>(&s_m[1][lr][32 * kt + 8 * lg]);
                if constexpr (KQ_LDS) {
                    ka[0] = *reinterpret_cast<const bf16x8*>(&s_k[b][16 * rt + lr][32 * kt + 8 * lg]);
                    qa[0] = *reinterpret_cast<const bf16x8*>(&s_q[16 * rt + lr][32 * kt + 8 * lg]);
                } else {
                    to_pieces(x.ka[i][kt], ka);
                    to_pieces(x.qa[i][kt], qa);
                }
                mfma_split_acc<NS, 2>(ka, mb, kacc[kt & 1]);
                mfma_split_acc<NS, 2>(qa, mb, qacc[kt & 1]);
            }
            floatx4 km = kacc[0][0], qq = qacc[0][0];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int pp = (j == 0 ? 1 : 0); pp < NP; ++pp) {
                    km += kacc[j][pp];
                    qq += qacc[j][pp];
                }
            qm[i] = qq;
            floatx4 xv;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                xv[e] = scal(x, b, i, e)[0] * raw_to_f32(x.vv[i][e]) - scal(x, b, i, e)[1] * km[e];
            put4(&s_x[0][lr][16 * rt + 4 * lg], &s_x[1][lr][16 * rt + 4 * lg], xv);
        }
        __syncthreads();
        // (2) U = T X; W = diag(r_k exp(gamma_C - gamma)) U
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = w + 4 * i;
            if (rt >= RT) continue;
            floatx4 uacc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int kt = 0; kt < KTC; ++kt) {
                if (32 * kt > 16 * rt + 15) continue;
                bf16x8 xb[2];
                xb[0] = *reinterpret_cast<const bf16x8*>(&s_x[0][lr][32 * kt + 8 * lg]);
                xb[1] = *reinterpret_cast<const bf16x8*>(&s_x[1][lr][32 * kt + 8 * lg]);
                mfma_split_acc<2, 2>(x.tf[i][kt], xb, uacc);
            }
            const floatx4 u = uacc[0] + uacc[1] + uacc[2];
            floatx4 wv;
#pragma unroll
            for (int e = 0; e < 4; ++e) wv[e] = scal(x, b, i, e)[3] * u[e];
            put4(&s_u[0][lr][16 * rt + 4 * lg], &s_u[1][lr][16 * rt + 4 * lg], u);
            put4(&s_w[0][lr][16 * rt + 4 * lg], &s_w[1][lr][16 * rt + 4 * lg], wv);
        }
        __syncthreads();
        // (3) O = diag(Gamma r_q) Q M0 + Ptil U
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = w + 4 * i;
            if (rt >= RT) continue;
            floatx4 oacc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int e = 0; e < 4; ++e) oacc[0][e] = scal(x, b, i, e)[2] * qm[i][e];
#pragma unroll
            for (int kt = 0; kt < KTC; ++kt) {
                if (32 * kt > 16 * rt + 15) continue;
                bf16x8 ub[2];
                ub[0] = *reinterpret_cast<const bf16x8*>(&s_u[0][lr][32 * kt + 8 * lg]);
                ub[1] = *reinterpret_cast<const bf16x8*>(&s_u[1][lr][32 * kt + 8 * lg]);
                mfma_split_acc<2, 2>(x.pf[i][kt], ub, oacc);
            }
            opend[i] = oacc[0] + oacc[1] + oacc[2];
        }
        // (4) M <- Gamma_C M + K^T W
#pragma unroll
        for (int i = 0; i < MTW; ++i) {
            const int mt = w + 4 * i;
            if (mt >= MT) continue;
            constexpr int NP = NS + 1;
            floatx4 acc[NP];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[0][e] = x.gc * macc[i][e];
#pragma unroll
            for (int pp = 1; pp < NP; ++pp) acc[pp] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < KTC; ++kt) {
                bf16x8 wb[2];
                wb[0] = *reinterpret_cast<const bf16x8*>(&s_w[0][lr][32 * kt + 8 * lg]);
                wb[1] = *reinterpret_cast<const bf16x8*>(&s_w[1][lr][32 * kt + 8 * lg]);
                if constexpr (KQ_LDS) {
                    // K^T fragment: feature 16 mt + lr, tokens 32 kt + 8 lg + e, read across
                    // the K rows in LDS (tokens past the chunk are zero rows).
                    bf16x8 ktf[1];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int tok = 32 * kt + 8 * lg + e;
                        ktf[0][e] = tok < C ? s_k[b][tok][16 * mt + lr] : (__bf16)0.f;
                    }
                    mfma_split_acc<1, 2>(ktf, wb, acc);
                } else {
                    mfma_split_acc<NS, 2>(x.kt[i][kt], wb, acc);
                }
            }
            floatx4 mnew = acc[0];
#pragma unroll
            for (int pp = 1; pp < NP; ++pp) mnew += acc[pp];
            macc[i] = mnew;
            store_m_lds(i, mt);
        }
    };

    // A full wait: nothing left in flight, so the compiler's wait bookkeeping starts clean
    // (no loop-carried loads that would force early waits inside the next chunk).
    auto settle = [&]() { __builtin_amdgcn_s_waitcnt(0); };

    if constexpr (C <= 64) {
        // Two operand sets alternate: the next chunk's operands load while this chunk
        // computes, and the wait for them lands at the end of the chunk.
        // Even chunks use LDS buffer 0, odd chunks buffer 1. Q and buffer (c + 1) & 1 are
        // last read by chunk c - 1 / before chunk c's first barrier, so they can be refilled
        // at the end of chunk c.
        R A, B;
        load(A, 0);
        store_kq(A, 0);
        settle();
        __syncthreads();
#pragma unroll 1
        for (int64_t c = 0; c < nch; c += 2) {
            load(B, c + 1);
            compute(A, 0);
            store_kq(B, 1);
            settle();
            __syncthreads();
            store_out(c);
            if (c + 1 >= nch) break;
            load(A, c + 2);
            compute(B, 1);
            store_kq(A, 0);
            settle();
            __syncthreads();
            store_out(c + 1);
        }
    } else {
        // Two sets of C = 128 operands do not fit the register file: load at the top.
        R A;
#pragma unroll 1
        for (int64_t c = 0; c < nch; ++c) {
            load(A, c);
            store_kq(A, (int)(c & 1));
            settle();
            __syncthreads();
            if (c > 0) store_out(c - 1);
            compute(A, (int)(c & 1));
            __syncthreads();
        }
        store_out(nch - 1);
    }

#pragma unroll
    for (int i = 0; i < MTW; ++i) {
        const int mt = w + 4 * i;
        if (mt >= MT) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            state_out[sbase + (int64_t)(16 * mt + 4 * lg + e) * D + cb * 16 + lr] = macc[i][e];
    }
}

template <int D, int C, typename TIn>
hipError_t launch_chunked_t(const Call& cl)
{
    constexpr bool F32IN = std::is_same<TIn, float>::value;
    const ChunkWs L = chunk_ws(cl.n, cl.t, cl.h_qk, cl.h_v, D, C, F32IN);
    char* ws = static_cast<char*>(cl.ws);
    const TIn* q = static_cast<const TIn*>(cl.q);
    const TIn* k = static_cast<const TIn*>(cl.k);
    const TIn* v = static_cast<const TIn*>(cl.v);
    const int64_t prep_blocks = cl.n * L.nch * cl.h_qk;
    hipLaunchKernelGGL((chunk_prep_kernel<D, C, TIn>), dim3((unsigned)prep_blocks), dim3(256), 0,
                       cl.stream, q, k, cl.g, cl.beta, ws, L, cl.t, cl.h_qk, cl.h_v, cl.eps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t scan_blocks = cl.n * cl.h_v * (D / 16);
    hipLaunchKernelGGL((chunk_scan_kernel<D, C, TIn>), dim3((unsigned)scan_blocks), dim3(256), 0,
                       cl.stream, q, k, v, ws, L, cl.state_in, cl.out, cl.state_out, cl.t,
                       cl.h_qk, cl.h_v, scan_blocks);
    return hipGetLastError();
}

template <int D, typename TIn>
hipError_t dispatch_c(const Call& cl, int chunk)
{
    switch (chunk) {
        case 16: return launch_chunked_t<D, 16, TIn>(cl);
        case 32: return launch_chunked_t<D, 32, TIn>(cl);
        case 64: return launch_chunked_t<D, 64, TIn>(cl);
        case 128: return launch_chunked_t<D, 128, TIn>(cl);
        default: return hipErrorInvalidValue;
    }
}

template <typename TIn>
hipError_t dispatch_d(const Call& cl, int chunk)
{
    switch (cl.d) {
        case 16: return dispatch_c<16, TIn>(cl, chunk);
        case 32: return dispatch_c<32, TIn>(cl, chunk);
        case 64: return dispatch_c<64, TIn>(cl, chunk);
        case 128: return dispatch_c<128, TIn>(cl, chunk);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t chunked_workspace_bytes(int64_t n, int64_t t, int32_t h_qk, int32_t h_v, int32_t d,
                               int chunk, int32_t dtype)
{
    return chunk_ws(n, t, h_qk, h_v, d, chunk, dtype != GDN_BF16).total;
}

hipError_t launch_chunked(const Call& c, int chunk)
{
    return c.dtype == GDN_BF16 ? dispatch_d<uint16_t>(c, chunk) : dispatch_d<float>(c, chunk);
}

}  // namespace gdn
