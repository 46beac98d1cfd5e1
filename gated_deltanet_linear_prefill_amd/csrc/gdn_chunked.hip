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
//   (I + A) U = diag(beta) (V - diag(Gamma) Khat M0),
//   A[r][s] = beta_r exp(gamma_r - gamma_s) khat_r . khat_s        (s < r)
// With T = (I + A)^-1 and K, Q the raw inputs, r_k, r_q their inverse norms:
//   U   = T' X,          T' = T diag(beta),   X = V - diag(a) (K M0),   a = Gamma r_k
//   O   = diag(o) (Q M0) + Ptil U,            o = Gamma r_q,
//         Ptil[r][s] = exp(gamma_r - gamma_s) r_q,r r_k,s q_r . k_s   (s <= r)
//   M_C = Gamma_C M0 + K^T diag(s) U,         s = r_k exp(gamma_C - gamma)
// The normalisation stays a diagonal scaling so the bf16 inputs enter the MFMAs exactly,
// and decays only appear as exp(gamma_r - gamma_s) with s <= r, so nothing overflows.
//
// Two kernels:
//  * chunk_prep_kernel (one workgroup per sequence, chunk and QK head; fully parallel):
//    inverse norms, gate prefix sums, the Gram matrices K K^T and Q K^T (MFMA, once per QK
//    head), then per V head A, T = (I + A)^-1 by blocked forward substitution in LDS, and
//    the per-token scalars. T' and Ptil go to the workspace as hi/lo bf16 MFMA A-operand
//    tiles (lower-triangular tiles only); for chunks of up to 32 tokens also the chunk
//    coupling H = K_next K^T diag(s) T' that the scan's chain recursion uses.
//  * chunk_scan_kernel (one workgroup per sequence, V head and 16 value channels;
//    sequential over chunks). For chunks of up to 32 tokens a chain wave runs the
//    recursion over the residuals X alone, state waves keep the state in MFMA accumulators
//    a chunk behind, and helper waves form the outputs and stage every input in LDS ahead of
//    use (the scan section below). Chunks of 64 and 128 tokens use a variant with two chain
//    waves that each hold half of the state and exchange one partial product per chunk.
//
// Operand order. Contractions over d_k and over chunk tokens both use k tiles of 32. The
// state's accumulator rows hold features in a permuted order (tile mt, row 4a + e holds
// feature 32 (mt >> 1) + 8 a + 4 (mt & 1) + e) and token k slots are permuted the same way
// (slot 8 lg + 4 h + e of token tile kt is token 32 kt + 16 h + 4 lg + e): then the four
// accumulator values a lane holds in two adjacent row tiles are exactly the eight k values
// that lane needs as a B operand, so U, W, X and the state feed the next MFMA from
// registers. Raw K and Q rows stay in natural feature order. The prepared A operands (T',
// Ptil, K^T) are written with the same token permutation.
//
// Precision: an MFMA operand that is not an exact bf16 input (the state, X, U, W, T',
// Ptil) is split into hi = bf16(x) and lo = bf16(x - hi) and multiplied as
// hi*hi + hi*lo + lo*hi (or hi + lo against an exact operand), which keeps about 16
// significant bits per operand with fp32 accumulation; one bf16 rounding would not meet the
// accuracy the recurrence needs (the page's "Keep the recurrent state on-chip" section keeps
// the state and gate in 32-bit floats for the same reason). Decay factors
// exp(gamma_r - gamma_s) <= 1 inside the C x C matrices use the hardware exponential
// (__expf); its relative error, a few 1e-6 at these arguments, is far below that precision.
// Where the gates allow it (none positive, spread at most SEP_SPAN over the chunk) each is
// formed as exp(gamma_r - gamma_b) exp(gamma_b - gamma_s) from per-token tables with an
// anchor b between s and r, which at most doubles that error.
#include <type_traits>

#include <atomic>

#include "gdn_internal.hpp"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// The same split for two values at once, each piece pair packed in one dword (the first
// value in the low half): one packed conversion gives both hi values, which are widened
// back with a shift and a mask.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t* hi, uint32_t* lo)
{
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{x0, x1}, bf16x2));
    const float h0 = __uint_as_float(h << 16), h1 = __uint_as_float(h & 0xffff0000u);
    *hi = h;
    *lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{x0 - h0, x1 - h1}, bf16x2));
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
// A and B enumerate k the same way, so any fixed relabelling of the 32 k slots applied to
// both operands leaves the product unchanged; the permutations below rely on that.

// Feature held by accumulator row rho (0..15) of state tile mt.
__host__ __device__ constexpr int feat_of(int mt, int rho)
{
    return 32 * (mt >> 1) + 8 * (rho >> 2) + 4 * (mt & 1) + (rho & 3);
}

// Chunk token in k slot 8 lg + j of token k tile kt.
__host__ __device__ constexpr int tok_of(int kt, int lg, int j)
{
    return 32 * kt + 16 * (j >> 2) + 4 * lg + (j & 3);
}

// Lower-triangular operand tiles are stored compactly: row tile rt (16 tokens) keeps the
// token k tiles 0 .. rt / 2, i.e. those that reach the diagonal. Index of (rt, 0):
__host__ __device__ constexpr int tri_off(int rt)
{
    return (rt / 2) * (rt / 2 + 1) + (rt & 1) * (rt / 2 + 1);
}

template <int D, int C, bool F32IN>
struct Geo {
    static constexpr int DP = D < 32 ? 32 : D;  // contraction over d, padded to k = 32
    static constexpr int CP = C < 32 ? 32 : C;  // contraction over chunk tokens, padded
    static constexpr int KTD = DP / 32;         // k tiles over d
    static constexpr int MTP = DP / 16;         // 16-row state tiles (padded features zero)
    static constexpr int KTC = CP / 32;         // k tiles over chunk tokens
    static constexpr int RT = C / 16;           // 16-token row tiles of a chunk
    static constexpr int NS = F32IN ? 2 : 1;    // bf16 pieces per q/k element
    static constexpr int NTRI = tri_off(RT);    // stored lower-triangular tiles
    static constexpr int NCH = KTD >= 2 ? 2 : 1;  // chain waves (split of d_k)
    static constexpr int KTH = KTD / NCH;       // d k tiles per chain wave
    static constexpr int MTH = 2 * KTH;         // state tiles per chain wave
    static constexpr int NOW = 4 - NCH;         // output waves
    static constexpr int RTO = (RT + NOW - 1) / NOW;  // row tiles per output wave
    static constexpr int NHF = RT * KTC;        // A fragments of the full C x C matrix H
    static constexpr bool WITH_H = C <= 32;     // H is prepared for the scan kernel that uses it
    static constexpr size_t TRI_BYTES = (size_t)NTRI * 2 * 1024;      // per (chunk, V head)
    static constexpr size_t H_BYTES = WITH_H ? (size_t)NHF * 2 * 1024 : 0;  // per (chunk, V head)
    static constexpr size_t SC_BYTES = (size_t)3 * CP * 4 + 16;       // per (chunk, V head)
};

// Workspace regions; every region starts 256-byte aligned.
struct ChunkWs {
    int64_t nch;                  // chunks per sequence
    size_t tt, pt, hh, sc, total; // byte offsets: T', Ptil, H, scalars
};

size_t align256(size_t x)
{
    return (x + 255) & ~size_t(255);
}

ChunkWs chunk_ws(int64_t n, int64_t t, int32_t h_qk, int32_t h_v, int32_t d, int chunk,
                 bool f32in)
{
    (void)d;
    (void)f32in;
    const int cp = chunk < 32 ? 32 : chunk;
    const size_t tri_bytes = (size_t)tri_off(chunk / 16) * 2 * 1024;
    const size_t h_bytes = chunk <= 32 ? (size_t)(chunk / 16) * (cp / 32) * 2 * 1024 : 0;
    const size_t sc_bytes = (size_t)3 * cp * 4 + 16;
    ChunkWs w;
    w.nch = (t + chunk - 1) / chunk;
    (void)h_qk;
    const size_t nv = (size_t)n * w.nch * h_v;
    w.tt = 0;
    w.pt = w.tt + align256(nv * tri_bytes);
    w.hh = w.pt + align256(nv * tri_bytes);
    w.sc = w.hh + align256(nv * h_bytes);
    w.total = w.sc + align256(nv * sc_bytes);
    return w;
}

// Raw fragment storage for prefetch registers: the loaded bits are kept as they arrive and
// turned into MFMA pieces at use, so issuing the next chunk's loads never has to wait.
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

__device__ __forceinline__ void to_pieces(const bf16x8& raw, bf16x8* piece)
{
    piece[0] = raw;
}

__device__ __forceinline__ void to_pieces(const floatx8& raw, bf16x8* piece)
{
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) split2(raw[2 * p], raw[2 * p + 1], &hi[p], &lo[p]);
    piece[0] = __builtin_bit_cast(bf16x8, u32x4{hi[0], hi[1], hi[2], hi[3]});
    piece[1] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], lo[2], lo[3]});
}

__device__ __forceinline__ bf16x8 buf_bf16x8(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ floatx4 buf_floatx4(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <typename TIn>
__device__ __forceinline__ TIn buf_elem(__amdgpu_buffer_rsrc_t r, int off);

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

// The same product with each split pass in its own accumulator (acc[0 .. NA + NB - 2]),
// so the passes do not wait on each other; the caller sums the accumulators at the end.
template <int NA, int NB>
__device__ __forceinline__ void mfma_split_acc(const bf16x8* a, const bf16x8* b, floatx4* acc)
{
    acc[0] = mfma_bf16(a[0], b[0], acc[0]);
    if constexpr (NB > 1) acc[1] = mfma_bf16(a[0], b[1], acc[1]);
    if constexpr (NA > 1) acc[NB] = mfma_bf16(a[1], b[0], acc[NB]);
}

// hi/lo B-fragment pieces of one k tile from the accumulators of its two row tiles.
__device__ __forceinline__ void pair_to_frag(const floatx4& a0, const floatx4& a1, bf16x8& hi,
                                             bf16x8& lo)
{
    uint32_t h[4], l[4];
    split2(a0[0], a0[1], &h[0], &l[0]);
    split2(a0[2], a0[3], &h[1], &l[1]);
    split2(a1[0], a1[1], &h[2], &l[2]);
    split2(a1[2], a1[3], &h[3], &l[3]);
    hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}

// Per-row-tile values (RT row tiles of 16 tokens, accumulator layout) as token k-tile
// B fragments; row tiles past the chunk (C = 16 pads to one k tile of 32) are zero.
template <int RT, int KTC>
__device__ __forceinline__ void rows_to_frags(const floatx4* rows, bf16x8 (*fr)[2])
{
#pragma unroll
    for (int kt = 0; kt < KTC; ++kt) {
        const floatx4 z = {0.f, 0.f, 0.f, 0.f};
        pair_to_frag(2 * kt < RT ? rows[2 * kt] : z, 2 * kt + 1 < RT ? rows[2 * kt + 1] : z,
                     fr[kt][0], fr[kt][1]);
    }
}

// Index of the t-th lower-triangular 16x16 tile (row tile >= column tile).
__device__ __forceinline__ void tri_tile(int t, int& rt, int& ct)
{
    rt = 0;
    while ((rt + 1) * (rt + 2) / 2 <= t) ++rt;
    ct = t - rt * (rt + 1) / 2;
}

// A workgroup barrier that waits only for this wave's LDS operations: the other waves see
// its LDS writes, while its global loads and stores may still be in flight. (__syncthreads()
// also waits for every outstanding global store and for loads that write LDS directly; the
// kernels wait for those explicitly where a result depends on them.)
__device__ __forceinline__ void barrier_lds_only()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// =============================================================================== prep
// Fragment index fi of a compact lower-triangular operand -> (row tile rt, k tile kt).
__device__ __forceinline__ void tri_frag(int fi, int& rt, int& kt)
{
    rt = 0;
    while (tri_off(rt + 1) <= fi) ++rt;
    kt = fi - tri_off(rt);
}

// Four waves per SIMD (registers for four resident workgroups per CU): the kernel is bound by
// latency, and the register allocation fits without spills. Phases are separated by barriers
// that wait for LDS only: nothing in the workgroup reads back the workspace it stores, so a
// phase never waits for the previous phase's stores to complete.
// Largest spread of a head's gate prefix sums over one chunk for which the prep kernel forms
// the pairwise decays as products of two exponentials: each factor then stays within
// [e^-60, e^60] (times an inverse norm of at most 1 / sqrt(eps)), far from fp32 overflow and
// underflow, while a chunk of 64 tokens at the workloads' gates spans about 8.
constexpr float SEP_SPAN = 60.f;

template <int D, int C, typename TIn, bool PH = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
chunk_prep_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const float* __restrict__ g,
                  const float* __restrict__ beta, char* __restrict__ ws, ChunkWs L, int64_t T,
                  int h_qk, int h_v, float eps, int stagger_wgs, int stagger_units)
{
    // Staggered start (stagger_units > 0: the whole grid resident at once, several workgroups
    // per CU). Every workgroup loads its q/k rows first and all would otherwise share the
    // memory bandwidth equally, so that none could start computing before nearly all rows
    // had arrived. Group i (workgroups i * stagger_wgs .. (i + 1) * stagger_wgs - 1, one per
    // CU) waits about the time one group's rows take to stream in, times i, so that earlier
    // groups compute while later groups' rows arrive.
    if (stagger_units > 0) {
        const int grp = (int)(blockIdx.x / (unsigned)stagger_wgs);
        for (int i = (grp * stagger_units) / 8; i > 0; --i) __builtin_amdgcn_s_sleep(8);
    }
    constexpr bool F32IN = std::is_same<TIn, float>::value;
    using G = Geo<D, C, F32IN>;
    constexpr int DP = G::DP, CP = G::CP, RT = G::RT, KTD = G::KTD, KTC = G::KTC;
    constexpr int NS = G::NS, NTRI = G::NTRI;
    constexpr int NB = RT;        // 16x16 diagonal blocks of T
    constexpr int KS = DP + 8;    // LDS row stride of the K / Q pieces (bf16)
    constexpr int CS = CP + 4;    // LDS row stride of the CP x CP fp32 matrices
    // The V heads of the QK head are taken NHP at a time, NWH waves each: for chunks of up to
    // 64 tokens two heads side by side (the diagonal solve needs one wave, the other writes
    // Ptil meanwhile), 128-token chunks one head with all four waves. For 64-token chunks T
    // is formed in place of A (INPLACE), so that both heads' matrices fit the LDS that four
    // resident workgroups per CU leave. PH (per head): one workgroup per (sequence, chunk, V
    // head) with all four waves on its head, each forming the QK head's Gram tiles again;
    // for grids that leave CUs idle, where a workgroup's latency rather than the chip's
    // throughput sets the time.
    static_assert(!PH || C == 64, "the per-head form is built for 64-token chunks");
    constexpr int NWH = PH || C > 64 ? 4 : 2;      // waves per V head
    constexpr int NHP = 4 / NWH;                   // V heads per pass
    constexpr bool INPLACE = C == 64 && !PH;
    constexpr size_t KQ_LDS = (size_t)2 * NS * CP * KS * 2;
    constexpr size_t AT_LDS = (size_t)NHP * (INPLACE ? 1 : 2) * CP * CS * 4;
    constexpr size_t U_LDS = KQ_LDS > AT_LDS ? KQ_LDS : AT_LDS;
    // The Gram tiles are shared by the V heads of a pass: every wave forms its share of them
    // once and writes A and Ptil for all NHP heads from it. The first NBW waves of each head
    // slot solve the diagonal blocks of T (one lane per column) while the others write Ptil,
    // so the Ptil fragments go to those others first (rank prk).
    constexpr int NFW = (NTRI + 3) / 4;  // Ptil fragments per wave
    constexpr int NBW = (NB * 16 + 63) / 64;
    constexpr int NNS = NHP * (NWH - NBW);  // waves that do not solve

    // The K and Q chunks (first phases) and the A / T matrices (later phases) share one
    // buffer; the Gram matrices live in registers in between.
    __shared__ __align__(16) char s_buf[U_LDS];
    __shared__ float s_rk[CP], s_rq[CP];
    __shared__ float s_gam[NHP][CP], s_beta[NHP][CP];
    __shared__ float s_sv[G::WITH_H ? NHP : 1][G::WITH_H ? CP : 1];  // s for H (chunks <= 32)
    __shared__ float s_x[4][16][17];  // per-wave 16x16 scratch (phase 6)
    __shared__ int s_sep[NHP];        // 1: the head's decays are formed as products (below)
    // Decay tables of the pass (phases 4 and 5), in the phase-6 scratch. In a tile pair
    // (row tile R, column tile S <= R) the anchor b = 16 R lies between every column token s
    // and row token r >= b, so exp(gamma_r - gamma_s) = exp(gamma_r - gamma_b) exp(gamma_b -
    // gamma_s). Per head slot: rho_k[r] = beta_r r_k,r exp(gamma_r - gamma_b(r)) and
    // rho_q[r] = r_q,r exp(gamma_r - gamma_b(r)) (CP each), then kappa[R][s] = r_k,s
    // exp(gamma_16R - gamma_s) for s < 16 R + 16 (packed by R: offset 8 R (R + 1)). An element
    // of A is then rho_k[r] kappa[R][s] (k_r . k_s) and one of Ptil rho_q[r] kappa[R][s]
    // (q_r . k_s). Used in the first pass when no gate of its heads is positive and each
    // head's gamma spans at most SEP_SPAN over the chunk, so that no factor overflows or
    // underflows where the product does not.
    constexpr int DSTR = 2 * CP + 8 * RT * (RT + 1);
    static_assert(NHP * DSTR + 16 <= 4 * 16 * 17, "decay tables (+16 floats read past the last "
                  "one, dropped by the selects) fit the phase-6 scratch");
    static_assert(64 * NWH >= CP, "one thread per token of a head slot");
    float* const s_dec = &s_x[0][0][0];
    auto s_kq = [&](int which, int part, int r, int f) -> __bf16& {
        return reinterpret_cast<__bf16*>(s_buf)[(((size_t)which * NS + part) * CP + r) * KS + f];
    };

    const int64_t nch = L.nch;
    const int unit = PH ? h_v : h_qk;  // workgroups per (sequence, chunk)
    const int hx = (int)(blockIdx.x % unit);
    const int64_t sc_idx = blockIdx.x / unit;
    const int64_t c = sc_idx % nch, seq = sc_idx / nch;
    const int hq = PH ? hx / (h_v / h_qk) : hx;
    const int64_t c0 = c * C;
    const int Cr = (int)((T - c0) < C ? (T - c0) : C);
    const int tid = threadIdx.x, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
    const int pm = w / NWH, wl = w % NWH;  // the head slot of this wave, its index there
    const int pt = tid - 64 * NWH * pm;    // thread index within the head slot
    const int prk = wl >= NBW ? pm * (NWH - NBW) + wl - NBW : NNS + pm * NBW + wl;
    const int grp = h_v / h_qk;
    const int npass = PH ? 1 : grp;  // V heads this workgroup takes, NHP per pass
    const int64_t tok0 = seq * T + c0;  // flattened token index of the chunk's first token
    float(*s_a)[CS] = reinterpret_cast<float(*)[CS]>(s_buf + (size_t)pm * (INPLACE ? 1 : 2) * CP * CS * 4);
    float(*s_t)[CS] = INPLACE ? s_a : reinterpret_cast<float(*)[CS]>(s_buf + ((size_t)pm * 2 + 1) * CP * CS * 4);
    // V head of slot p in the pass starting at head g0 (a slot past the QK head's V heads
    // repeats the pass's first head: the same values are computed and written twice)
    auto head_at = [&](int g0, int p) { return PH ? hx : hq * grp + (g0 + p < grp ? g0 + p : g0); };
    auto head_of = [&](int g0) { return head_at(g0, pm); };
    auto a_of = [&](int p) {
        return reinterpret_cast<float(*)[CS]>(s_buf + (size_t)p * (INPLACE ? 1 : 2) * CP * CS * 4);
    };

    // Gate and write strength of one V head for this chunk (the first wave of each head
    // slot; E tokens per lane), loaded one pass ahead of their use.
    constexpr int E = (CP + 63) / 64;
    float gv[E], bv[E];
    auto load_gb = [&](int hv) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = l * E + e;
            const bool ok = i < Cr;
            const int64_t off = (tok0 + (ok ? i : 0)) * h_v + hv;
            const float g_in = g[off], b_in = beta[off];
            gv[e] = ok ? g_in : 0.f;
            bv[e] = ok ? b_in : 0.f;
        }
    };
    if (wl == 0) load_gb(head_of(0));

    // Gate prefix sums gamma and write strengths of the pass starting at V head g0 into
    // LDS (the first wave of each head slot); the next pass's gates are loaded meanwhile.
    auto gate_prefix = [&](int g0) {
        if (wl != 0) return;
        float run = 0.f, gs[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            run += gv[e];
            gs[e] = run;
        }
        float x = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (l >= off) x += y;
        }
        const float excl = x - run;
        bool nonpos = true;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = l * E + e;
            if (i < CP) {
                s_gam[pm][i] = gs[e] + excl;
                s_beta[pm][i] = bv[e];
            }
            nonpos = nonpos && gv[e] <= 0.f;  // false for NaN
        }
        // With no positive gate gamma falls from g_0 (lane 0) to the total (lane 63), so that
        // difference is its spread over the chunk (NaN or infinite for such gates: no product
        // form then).
        const bool mono = __ballot(!nonpos) == 0;
        const float spread = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gs[0] + excl))) -
                             __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
        if (l == 0) s_sep[pm] = mono && spread <= SEP_SPAN ? 1 : 0;
        if (g0 + NHP < npass) load_gb(head_of(g0 + NHP));
    };

    // The decay tables of this head slot's head in the first pass (gamma, beta and the
    // inverse norms in LDS); every thread of the slot forms rho for one token and kappa for
    // every R of its residue class.
    auto build_dec = [&]() {
        float* d = s_dec + pm * DSTR;
        if (pt < CP) {
            const float e = __expf(s_gam[pm][pt] - s_gam[pm][pt & ~15]);
            d[pt] = s_beta[pm][pt] * s_rk[pt] * e;
            d[CP + pt] = s_rq[pt] * e;
        }
        constexpr int SL = 64 * NWH / CP;
        const int sv = pt % CP, rg = pt / CP;
#pragma unroll
        for (int j = 0; j < (RT + SL - 1) / SL; ++j) {
            const int R = rg + SL * j;
            if (R < RT && sv < 16 * R + 16)
                d[2 * CP + 8 * R * (R + 1) + sv] = s_rk[sv] * __expf(s_gam[pm][16 * R] - s_gam[pm][sv]);
        }
    };
    // Whether every head of the pass takes the product form (wave-uniform).
    auto sep_pass = [&]() {
        int all = 1;
#pragma unroll
        for (int p = 0; p < NHP; ++p) all &= s_sep[p];
        return __builtin_amdgcn_readfirstlane(all) != 0;
    };

    // The next chunk's key rows for H (see below), loaded now so that they arrive while the
    // chunk's own rows are loaded and normalised.
    constexpr int NIT = G::WITH_H ? (RT + NWH - 1) / NWH : 0;
    using Raw = typename RawFrag<TIn>::type;
    Raw bnr[NIT > 0 ? NIT : 1][KTD];
    if constexpr (G::WITH_H) {
        const int64_t rows_next = T - (c0 + C) < C ? T - (c0 + C) : (int64_t)C;  // may be <= 0
        const TIn* kn = k + ((tok0 + C) * h_qk + hq) * (int64_t)D;
        const auto r = make_rsrc(rows_next > 0 ? kn : k, rows_next > 0 ? (rows_next - 1) * h_qk * D * (int64_t)sizeof(TIn) + D * (int64_t)sizeof(TIn) : 0);
#pragma unroll
        for (int i = 0; i < NIT; ++i) {
            const int it = wl + NWH * i;
#pragma unroll
            for (int kt = 0; kt < KTD; ++kt) {
                const int f = 32 * kt + 8 * lg;
                const int off = ((16 * it + lr) * h_qk * D + f) * (int)sizeof(TIn);
                bnr[i][kt] = buf_raw_frag<TIn>(r, f < D && it < RT ? off : (int)OOR);
            }
        }
    }

    // ---- phase 0: inverse norms of the q and k rows; both chunks into LDS as bf16 pieces
    //      (rows past the chunk and padded features are zero). The loads of a batch of
    //      rows are all issued before any of them is used. The first pass's gate prefix
    //      sums are formed here too, while the rows arrive.
    {
        constexpr int EPL = D / 16;  // elements per lane, 16 lanes per row
        constexpr int NPASS = CP / 16;
        constexpr int BATCH = NPASS < 4 ? NPASS : 4;
        const int sub = tid & 15;
        // bf16 rows of 128 features: each thread's 8 features are one 16-byte load, copied to
        // LDS as loaded (a bf16 input is its own hi piece); the norms square the widened
        // values in the same order as the general path below.
        constexpr bool RAW16 = std::is_same<TIn, uint16_t>::value && NS == 1 && D == DP && EPL == 8;
        if constexpr (RAW16) {
#pragma unroll
            for (int p0 = 0; p0 < NPASS; p0 += BATCH) {
                u32x4 qr[BATCH], kr[BATCH];
#pragma unroll
                for (int b = 0; b < BATCH; ++b) {
                    const int r = 16 * (p0 + b) + (tid >> 4);
                    const bool ok = r < Cr;
                    const int64_t off = ((tok0 + (ok ? r : 0)) * h_qk + hq) * (int64_t)D + sub * EPL;
                    qr[b] = *reinterpret_cast<const u32x4*>(q + off);
                    kr[b] = *reinterpret_cast<const u32x4*>(k + off);
                }
                float sq[BATCH], sk[BATCH];
#pragma unroll
                for (int b = 0; b < BATCH; ++b) {
                    const int r = 16 * (p0 + b) + (tid >> 4);
                    const bool ok = r < Cr;
                    float qq = 0.f, kk = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float q0 = __uint_as_float(qr[b][e] << 16), q1 = __uint_as_float(qr[b][e] & 0xffff0000u);
                        const float k0 = __uint_as_float(kr[b][e] << 16), k1 = __uint_as_float(kr[b][e] & 0xffff0000u);
                        qq += q0 * q0;
                        qq += q1 * q1;
                        kk += k0 * k0;
                        kk += k1 * k1;
                    }
                    sq[b] = row16_sum(qq);
                    sk[b] = row16_sum(kk);
                    const u32x4 z = {0u, 0u, 0u, 0u};
                    *reinterpret_cast<u32x4*>(&s_kq(0, 0, r, sub * EPL)) = ok ? kr[b] : z;
                    *reinterpret_cast<u32x4*>(&s_kq(1, 0, r, sub * EPL)) = ok ? qr[b] : z;
                }
                // The 16 lanes of a row group hold the same 2 x BATCH sums: lane sub < 2 BATCH
                // forms inverse norm number sub (q rows first, then k rows), one per lane.
                static_assert(2 * BATCH <= 16, "one inverse norm per lane of a row group");
                const int bs = sub % BATCH;
                float xq = sq[0], xk = sk[0];
#pragma unroll
                for (int b = 1; b < BATCH; ++b) {
                    xq = bs == b ? sq[b] : xq;
                    xk = bs == b ? sk[b] : xk;
                }
                const float rinv = 1.0f / sqrtf((sub < BATCH ? xq : xk) + eps);
                if (sub < 2 * BATCH) {
                    const int r = 16 * (p0 + bs) + (tid >> 4);
                    const float val = r < Cr ? rinv : 0.f;
                    if (sub < BATCH) s_rq[r] = val;
                    else s_rk[r] = val;
                }
            }
        }
#pragma unroll
        for (int p0 = 0; p0 < (RAW16 ? 0 : NPASS); p0 += BATCH) {
            float qv[BATCH][EPL], kv[BATCH][EPL];
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
                const int r = 16 * (p0 + b) + (tid >> 4);
                const bool ok = r < Cr;
                const int64_t off = ((tok0 + (ok ? r : 0)) * h_qk + hq) * (int64_t)D + sub * EPL;
                load_n<EPL>(q + off, qv[b]);
                load_n<EPL>(k + off, kv[b]);
            }
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
                const int r = 16 * (p0 + b) + (tid >> 4);
                const bool ok = r < Cr;
                float qq = 0.f, kk = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    qq += qv[b][e] * qv[b][e];
                    kk += kv[b][e] * kv[b][e];
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
                    split_bf16(ok ? kv[b][e] : 0.f, hi, lo);
                    s_kq(0, 0, r, sub * EPL + e) = hi;
                    if constexpr (NS > 1) s_kq(0, 1, r, sub * EPL + e) = lo;
                    split_bf16(ok ? qv[b][e] : 0.f, hi, lo);
                    s_kq(1, 0, r, sub * EPL + e) = hi;
                    if constexpr (NS > 1) s_kq(1, 1, r, sub * EPL + e) = lo;
                }
                if constexpr (D < DP) {  // zero the padded features
#pragma unroll
                    for (int e = 0; e < (DP - D) / 16; ++e)
#pragma unroll
                        for (int which = 0; which < 2; ++which)
#pragma unroll
                            for (int part = 0; part < NS; ++part)
                                s_kq(which, part, r, D + sub * ((DP - D) / 16) + e) = (__bf16)0.f;
                }
            }
        }
    }
    gate_prefix(0);
    barrier_lds_only();

    // ---- phase 2: Gram matrices from the raw inputs, kept in registers for every V head
    //      of this QK head.
    //  * K K^T, lower 16x16 tiles (rt >= ct), accumulator rows r, columns s: for A.
    //  * K Q^T, the tile pairs (2 kt, rt), (2 kt + 1, rt) behind Ptil^T fragment (rt, kt):
    //    accumulator rows are tokens s of K, columns tokens r of Q, so the four values a
    //    lane holds in the two tiles are the eight k slots (permuted token order) of the
    //    B fragment of Ptil^T the scan kernel multiplies U^T with.
    build_dec();  // first pass; visible after the barrier that ends phase 2
    constexpr int NTL = RT * (RT + 1) / 2;
    constexpr int NTW = (NTL + 3) / 4;  // K K^T tiles per wave
    constexpr int NPG = NS == 1 ? 1 : 3; // split passes of a Gram product
    // Gram tile: rows of chunk `wa` (0 = K, 1 = Q) tile ta against rows of chunk `wb` tile tb.
    auto gram = [&](int wa, int ta, int wb, int tb) {
        floatx4 acc[NPG];
#pragma unroll
        for (int p = 0; p < NPG; ++p) acc[p] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < KTD; ++kt) {
            bf16x8 a[NS], b[NS];
#pragma unroll
            for (int part = 0; part < NS; ++part) {
                a[part] = *reinterpret_cast<const bf16x8*>(&s_kq(wa, part, 16 * ta + lr, 32 * kt + 8 * lg));
                b[part] = *reinterpret_cast<const bf16x8*>(&s_kq(wb, part, 16 * tb + lr, 32 * kt + 8 * lg));
            }
            mfma_split_acc<NS, NS>(a, b, acc);
        }
        floatx4 s = acc[0];
#pragma unroll
        for (int p = 1; p < NPG; ++p) s += acc[p];
        return s;
    };
    floatx4 gk[NTW];
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        gk[i] = floatx4{0.f, 0.f, 0.f, 0.f};
        const int ti = w + 4 * i;
        if (ti < NTL) {
            int rt, ct;
            tri_tile(ti, rt, ct);
            gk[i] = gram(0, rt, 0, ct);
        }
    }
    floatx4 gp[NFW][2];  // K Q^T tile pairs of this wave's Ptil fragments
#pragma unroll
    for (int i = 0; i < NFW; ++i) {
        gp[i][0] = gp[i][1] = floatx4{0.f, 0.f, 0.f, 0.f};
        const int fi = prk + 4 * i;
        if (fi < NTRI) {
            int rt, kt;
            tri_frag(fi, rt, kt);
            gp[i][0] = gram(0, 2 * kt, 1, rt);
            if (2 * kt + 1 <= rt) gp[i][1] = gram(0, 2 * kt + 1, 1, rt);
        }
    }
    // K_c K_{c+1}^T against the next chunk's keys (zero past the sequence), for
    // H = K_{c+1} K_c^T diag(s) T': wave wl of a head slot takes the rows of H in row tiles
    // it = wl, wl + NWH, ...
    // The tile pairs over K_c's tokens m are kept as B fragments (k slots m in the permuted
    // token order, columns the tokens i of chunk c + 1).
    bf16x8 gnb[NIT > 0 ? NIT : 1][KTC][2];
    if constexpr (G::WITH_H) {
#pragma unroll
        for (int i = 0; i < NIT; ++i) {
            const int it = wl + NWH * i;
            floatx4 gt[2 * KTC];
#pragma unroll
            for (int mt = 0; mt < 2 * KTC; ++mt) gt[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
            if (it < RT) {
                bf16x8 bn[KTD][NS];
#pragma unroll
                for (int kt = 0; kt < KTD; ++kt) to_pieces(bnr[i][kt], bn[kt]);
#pragma unroll
                for (int mt = 0; mt < RT; ++mt) {
                    floatx4 acc[NPG];
#pragma unroll
                    for (int p = 0; p < NPG; ++p) acc[p] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kt = 0; kt < KTD; ++kt) {
                        bf16x8 a[NS];
#pragma unroll
                        for (int part = 0; part < NS; ++part)
                            a[part] = *reinterpret_cast<const bf16x8*>(&s_kq(0, part, 16 * mt + lr, 32 * kt + 8 * lg));
                        mfma_split_acc<NS, NS>(a, bn[kt], acc);
                    }
                    gt[mt] = acc[0];
#pragma unroll
                    for (int p = 1; p < NPG; ++p) gt[mt] += acc[p];
                }
            }
#pragma unroll
            for (int kt = 0; kt < KTC; ++kt) pair_to_frag(gt[2 * kt], gt[2 * kt + 1], gnb[i][kt][0], gnb[i][kt][1]);
        }
    }
    barrier_lds_only();  // the K / Q buffer becomes A / T below

    for (int g0 = 0; g0 < npass; g0 += NHP) {
        const int hv = head_of(g0);
        const int64_t vh = (seq * nch + c) * h_v + hv;

        // ---- phase 3 (passes after the first; the first pass's ran in phase 0)
        if (g0 > 0) {
            gate_prefix(g0);
            barrier_lds_only();
        }
        // the tables are built for the first pass only (in phase 2); later passes, for more
        // than NHP V heads per QK head, form every decay as one exponential
        const bool sep = g0 == 0 && sep_pass();

        // ---- per-token scalars a = Gamma r_k, s = r_k exp(gamma_C - gamma), o = Gamma r_q
        //      and Gamma_C (padded tokens carry r_k = r_q = 0, so their scalars are zero)
        {
            float* scp = reinterpret_cast<float*>(ws + L.sc + (size_t)vh * G::SC_BYTES);
            const float gam_c = s_gam[pm][CP - 1];  // padded tokens add g = 0
            if (pt < CP) {
                const int i = pt;
                const float Gi = expf(s_gam[pm][i]);
                const float si = s_rk[i] * expf(gam_c - s_gam[pm][i]);
                scp[i] = Gi * s_rk[i];
                scp[CP + i] = si;
                scp[2 * CP + i] = Gi * s_rq[i];
                if constexpr (G::WITH_H) s_sv[pm][i] = si;  // for H below
            }
            if (pt == 0) scp[3 * CP] = expf(gam_c);
        }

        // ---- phase 4: A = strictly lower (beta_r exp(gamma_r - gamma_s) r_k,r r_k,s k_r . k_s)
        //      for every V head of the pass
        if (sep) {
#pragma unroll
            for (int i = 0; i < NTW; ++i) {
                const int ti = w + 4 * i;
                if (ti < NTL) {
                    int rt, ct;
                    tri_tile(ti, rt, ct);
#pragma unroll
                    for (int p = 0; p < NHP; ++p) {
                        float(*s_ap)[CS] = a_of(p);
                        const float* d = s_dec + p * DSTR;
                        const int s = 16 * ct + lr;
                        const float kap = d[2 * CP + 8 * rt * (rt + 1) + s];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 16 * rt + 4 * lg + e;
                            const float a = d[r] * kap * gk[i][e];
                            s_ap[r][s] = s < r ? a : 0.f;
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NTW; ++i) {
                const int ti = w + 4 * i;
                if (ti < NTL) {
                    int rt, ct;
                    tri_tile(ti, rt, ct);
#pragma unroll
                    for (int p = 0; p < NHP; ++p) {
                        float(*s_ap)[CS] = a_of(p);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 16 * rt + 4 * lg + e, s = 16 * ct + lr;
                            // formed for every element and selected (above the diagonal the
                            // decay may overflow; the select drops it)
                            const float a = s_beta[p][r] * __expf(s_gam[p][r] - s_gam[p][s]) * s_rk[r] * s_rk[s] * gk[i][e];
                            s_ap[r][s] = s < r ? a : 0.f;
                        }
                    }
                }
            }
        }
        barrier_lds_only();

        // ---- phase 5: diagonal 16x16 blocks of T by forward substitution, one lane per
        //      column: T[r][s] = delta_rs - sum_{m<r} A[r][m] T[m][s]; then (the other waves
        //      at once) Ptil^T of every V head of the pass as B fragments (rt, kt), hi and lo:
        //      slot 4 h + e holds Ptil[16 rt + lr][16 (2 kt + h) + 4 lg + e], which is zero
        //      above the diagonal.
        if (pt < NB * 16) {
            const int b = pt >> 4, s = pt & 15;
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
#pragma unroll
        for (int i = 0; i < NFW; ++i) {
            const int fi = prk + 4 * i;
            if (fi >= NTRI) continue;
            int rt, kt;
            tri_frag(fi, rt, kt);
            const int r = 16 * rt + lr;
#pragma unroll
            for (int p = 0; p < NHP; ++p) {
                const int64_t vhp = (seq * nch + c) * h_v + head_at(g0, p);
                char* pt_base = ws + L.pt + (size_t)vhp * G::TRI_BYTES;
                float val[8];
                if (sep) {
                    const float* d = s_dec + p * DSTR;
                    const float rho = d[CP + r];
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            // past the row tile (zero Gram tiles) kappa is read from the next
                            // R's entries or the slack after the tables; the select drops it
                            const int s = 32 * kt + 16 * h + 4 * lg + e;
                            const float pv = rho * d[2 * CP + 8 * rt * (rt + 1) + s] * gp[i][h][e];
                            val[4 * h + e] = s <= r ? pv : 0.f;
                        }
                } else {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int s = 32 * kt + 16 * h + 4 * lg + e;
                            const float pv = __expf(s_gam[p][r] - s_gam[p][s]) * s_rq[r] * s_rk[s] * gp[i][h][e];
                            val[4 * h + e] = s <= r ? pv : 0.f;
                        }
                }
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) split2(val[2 * q2], val[2 * q2 + 1], &hi[q2], &lo[q2]);
                *reinterpret_cast<u32x4*>(pt_base + (size_t)(2 * fi) * 1024 + l * 16) = u32x4{hi[0], hi[1], hi[2], hi[3]};
                *reinterpret_cast<u32x4*>(pt_base + (size_t)(2 * fi + 1) * 1024 + l * 16) = u32x4{lo[0], lo[1], lo[2], lo[3]};
            }
        }
        barrier_lds_only();

        // ---- phase 6: off-diagonal blocks, block row by block row:
        //      T_ij = -T_ii (sum_{m=j}^{i-1} A_im T_mj)   (fp32 MFMA)
        auto offdiag = [&](int i, int j) {
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
            return y;
        };
        if constexpr (INPLACE) {
            // T_ij replaces A_ij, which the other blocks of row i still read: every wave forms
            // its blocks of the row first, and writes them after a barrier.
            constexpr int NJ = (NB + NWH - 1) / NWH;
#pragma unroll 1
            for (int i = 1; i < NB; ++i) {
                floatx4 yv[NJ];
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj)
                    if (wl + NWH * jj < i) yv[jj] = offdiag(i, wl + NWH * jj);
                barrier_lds_only();
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj) {
                    const int j = wl + NWH * jj;
                    if (j < i) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) s_t[16 * i + 4 * lg + e][16 * j + lr] = -yv[jj][e];
                    }
                }
                barrier_lds_only();
            }
        } else {
            for (int i = 1; i < NB; ++i) {
                for (int j = wl; j < i; j += NWH) {
                    const floatx4 y = offdiag(i, j);
#pragma unroll
                    for (int e = 0; e < 4; ++e) s_t[16 * i + 4 * lg + e][16 * j + lr] = -y[e];
                    lds_fence();
                }
                barrier_lds_only();
            }
        }

        // ---- T' = T diag(beta) as compact hi/lo A-operand tiles with the permuted token
        //      order in k
        {
            char* tt_base = ws + L.tt + (size_t)vh * G::TRI_BYTES;
            for (int fi = wl; fi < NTRI; fi += NWH) {
                int rt, kt;
                tri_frag(fi, rt, kt);
                const int r = 16 * rt + lr;
                float val[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int s = tok_of(kt, lg, j);
                    const float tv = s_t[r][s] * s_beta[pm][s];  // above the diagonal: dropped
                    val[j] = s <= r ? tv : 0.f;
                }
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) split2(val[2 * p], val[2 * p + 1], &hi[p], &lo[p]);
                *reinterpret_cast<u32x4*>(tt_base + (size_t)(2 * fi) * 1024 + l * 16) = u32x4{hi[0], hi[1], hi[2], hi[3]};
                *reinterpret_cast<u32x4*>(tt_base + (size_t)(2 * fi + 1) * 1024 + l * 16) = u32x4{lo[0], lo[1], lo[2], lo[3]};
            }
        }

        // ---- H = K_{c+1} K_c^T diag(s) T' as A fragments (rows: tokens of chunk c + 1, k slots:
        //      tokens of chunk c, permuted order), formed transposed: H^T = (diag(s) T')^T G^T
        //      with G^T's B fragments from above. The A operand (diag(s) T')^T holds, for row
        //      j and k slot of token m, s_m T[m][j] beta_j (zero for m < j), whose fragments
        //      have the same registers as the B fragments of diag(s) T'.
        if constexpr (G::WITH_H) {
            char* hh_base = ws + L.hh + (size_t)vh * G::H_BYTES;
#pragma unroll
            for (int i = 0; i < NIT; ++i) {
                const int it = wl + NWH * i;
                if (it >= RT) continue;
                floatx4 ht[2 * KTC];  // H^T tiles (jt, it)
#pragma unroll
                for (int jt = 0; jt < 2 * KTC; ++jt) {
                    ht[jt] = floatx4{0.f, 0.f, 0.f, 0.f};
                    if (jt >= RT) continue;
#pragma unroll
                    for (int kt = 0; kt < KTC; ++kt) {
                        if (32 * kt + 31 < 16 * jt) continue;  // all m < j: zero block
                        const int j = 16 * jt + lr;
                        float val[8];
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const int m = tok_of(kt, lg, q);
                            val[q] = (m >= j && m < C) ? s_sv[pm][m] * s_t[m][j] * s_beta[pm][j] : 0.f;
                        }
                        uint32_t hi[4], lo[4];
#pragma unroll
                        for (int p = 0; p < 4; ++p) split2(val[2 * p], val[2 * p + 1], &hi[p], &lo[p]);
                        const bf16x8 a[2] = {__builtin_bit_cast(bf16x8, u32x4{hi[0], hi[1], hi[2], hi[3]}),
                                             __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], lo[2], lo[3]})};
                        ht[jt] = mfma_split<2, 2>(a, gnb[i][kt], ht[jt]);
                    }
                }
#pragma unroll
                for (int kt = 0; kt < KTC; ++kt) {
                    bf16x8 hi, lo;
                    pair_to_frag(ht[2 * kt], ht[2 * kt + 1], hi, lo);
                    const int fi = it * KTC + kt;
                    *reinterpret_cast<bf16x8*>(hh_base + (size_t)(2 * fi) * 1024 + l * 16) = hi;
                    *reinterpret_cast<bf16x8*>(hh_base + (size_t)(2 * fi + 1) * 1024 + l * 16) = lo;
                }
            }
        }
        barrier_lds_only();  // s_a, s_t and the gate prefix sums are rewritten for the next V head
    }
}

// =============================================================================== scan
// Scan workgroup (chunks of up to 32 tokens): one "chain" wave, NSW "state" waves and
// "helper" waves (one output helper per 16-token row tile, three staging helpers).
//
// The recursion the chain wave runs involves only X, the residuals V - diag(a) K M of a
// chunk:
//   X_{c+1} = V_{c+1} - diag(a_{c+1}) (Gamma_c P_{c+1} + H_c X_c),
//   P_{c+1} = K_{c+1} M_c,     H_c = K_{c+1} K_c^T diag(s_c) T'_c  (prepared per chunk),
// since K_{c+1} M_{c+1} = Gamma_c K_{c+1} M_c + K_{c+1} K_c^T W_c and W_c = diag(s_c) T'_c X_c.
// P_{c+1} needs the state of one chunk earlier, so the state waves, which hold the state
// split over d_k, form it (with the reduction over d_k) a chunk before it is used: no
// exchange over d_k sits on the chain's path. The chain wave also forms U = T' X and
// W = diag(s) U; the state waves apply M_{c+1} = Gamma_c M_c + K_c^T W_c one chunk later and
// form their parts of Q_{c+1} M_{c+1}, and the first helpers complete the outputs
// O_c = diag(o) Q_c M_c + Ptil_c U_c.
//
// The other helpers move every input into LDS two windows ahead of its use, with loads
// that write LDS directly (each lane's 16 bytes land at the destination base plus 16 bytes
// per lane): global loads are the scarce resource here, and this way the data never passes
// through registers. K and Q arrive as whole token rows (a load whose lanes cover 16 rows of
// 64 bytes, the MFMA fragment shape of a bf16 row, runs at about a third of the rate of one
// covering whole 128-byte lines), with their 16-byte granules swizzled so that fragment and
// transposing reads of the same copy are free of bank conflicts. fp32 rows (which are split
// into bf16 hi/lo planes) and d = 16 rows (shorter than a staged row) go through registers.
//
// Time advances in windows c = -2, -1, ..., nch - 1 (and one idle window more when that
// count is odd, so that the two-window loops below have no conditional half), each opened
// by a workgroup barrier:
//   chain    window c: X_{c+1}, U_{c+1}, W_{c+1} (c >= -1); H_{c+1} X_{c+1}; reads the
//                      V block, scalars and T' of chunk c + 2
//   state    window c: M_{c+1} (c >= 0); (Q_{c+1} M_{c+1})^T; Gamma_{c+1} P_{c+2} and
//                      K_{c+2}^T fragments
//   output   window c: outputs of chunk c                 (c >= 0)
//   staging  window c: issue K_{c+4}, T', V and scalars of chunk c + 4, H_{c+3}, Q_{c+3},
//                      Ptil_{c+2}; wait for those issued in window c - 1
// Staged inputs sit in rings of three chunks (the scalars in eight); exchanges between the
// compute waves are double-buffered by chunk parity.
template <int D, int C, typename TIn>
struct ScanGeo {
    static_assert(C <= 32, "longer chunks use the wide-chunk kernel");
    using G = Geo<D, C, std::is_same<TIn, float>::value>;
    static constexpr int ES = sizeof(TIn);
    static constexpr int NSW = G::KTD >= 2 ? 2 : 1;       // state waves
    static constexpr int KPS = G::KTD / NSW;               // d_k tiles per state wave
    static constexpr int NOH = G::RT;                      // output helpers, one row tile each
    static constexpr int NSH = 3;                          // staging helpers
    static constexpr int NHW = NOH + NSH;                  // helper waves
    static constexpr int THREADS = 64 * (1 + NSW + NHW);
    static constexpr int NR = 3;                           // ring depth of the staged inputs
    // Staged rows: one bf16 piece of DP features in 16-byte granules; granule j of row r sits
    // at position j ^ swz(r).
    static constexpr int ROWB = G::DP * 2;                 // bytes per staged row
    static constexpr int RPB = 256 / ROWB;                 // staged rows per 64 LDS banks
    static constexpr int NG = ROWB / 16;                   // granules per staged row
    // Raw q/k rows: RB bytes, loaded as LPR lanes of 16 bytes, RPI rows per instruction.
    static constexpr int RB = D * ES;
    static constexpr int LPR = RB / 16;
    static constexpr int RPI = 64 / LPR;
    static constexpr int NKI = (C + RPI - 1) / RPI;        // row loads per chunk
    // K and Q rows load straight into LDS when a load's 64 lanes fill 1 KB of staged rows
    // (bf16 and d >= 32); otherwise they go through registers.
    static constexpr bool DQK = ES == 2 && D >= 32;
    // Q ring depth: rows loaded straight into LDS are issued two windows before use (three
    // slots); rows written from registers one window before (two slots).
    static constexpr int NRQ = DQK ? NR : 2;
    // The V block (16 channels of a token): bf16 rows straight into LDS (read back with
    // transposing reads); fp32 through registers, transposed to channel-major.
    static constexpr bool DV = ES == 2;
    static constexpr int LPT = ES;                         // lanes per token of a V load
    static constexpr int TPI = 64 / LPT;                   // tokens per V load
    static constexpr int NVI = (C + TPI - 1) / TPI;
    static constexpr int VS = G::CP + 4;                   // LDS row stride of a transposed V block
    static constexpr size_t K_BYTES = (size_t)G::NS * G::CP * ROWB;
    static constexpr size_t Q_BYTES = K_BYTES;
    static constexpr size_t V_BYTES = DV ? (size_t)G::CP * 32 : (size_t)16 * VS * 4;
};

// Granule swizzle of the staged rows. A fragment read (16 consecutive rows, one granule)
// and a transposing read (4 consecutive rows x 4 consecutive granules per 16 lanes) then
// each touch 16 distinct 16-byte bank groups.
template <int RPB>
__device__ __forceinline__ int swz(int r)
{
    return ((r >> 2) & 3) | (((r & 3) / RPB) << 2);
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (gfx950 ds_read_b64_tr_b16). Within each 16-lane group, output lane j
// receives in slot p element (j mod 4) of the 8 bytes addressed by lane 4 p + j / 4 of the
// group (established with an in-bounds probe of the instruction).
__device__ __forceinline__ bf16x4 lds_read_tr16(const void* p)
{
    typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf16;
    const v4bf16 r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) v4bf16*)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// A 16-byte-per-lane buffer load that writes LDS directly: lane l's bytes land at
// lds + 16 l (established with an in-bounds probe of the instruction).


// Calls f(std::integral_constant<int, i>) for the wave-uniform index i in [I, N), so that the
// callee is specialised for each index.
template <int I, int N, typename F>
__device__ __forceinline__ void dispatch_index(int i, F&& f)
{
    if constexpr (I < N) {
        if (i == I) f(std::integral_constant<int, I>{});
        else dispatch_index<I + 1, N>(i, f);
    }
}

// Wait until at most n vector memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int D, int C, typename TIn>
__global__ void __launch_bounds__((ScanGeo<D, C, TIn>::THREADS)) __attribute__((amdgpu_waves_per_eu(1, 2)))
chunk_scan_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
                  const char* __restrict__ ws, ChunkWs L, const float* state_in,
                  float* __restrict__ out, float* state_out, int64_t T, int h_qk, int h_v,
                  int64_t nblocks)
{
    constexpr bool F32IN = std::is_same<TIn, float>::value;
    using G = Geo<D, C, F32IN>;
    using SG = ScanGeo<D, C, TIn>;
    constexpr int CP = G::CP, RT = G::RT, KTC = G::KTC, NS = G::NS;
    constexpr int NTRI = G::NTRI, NHF = G::NHF;
    constexpr int NSW = SG::NSW, KPS = SG::KPS, NHW = SG::NHW, NOH = SG::NOH, NSH = SG::NSH;
    constexpr int NR = SG::NR, ROWB = SG::ROWB, RPB = SG::RPB, NG = SG::NG;
    constexpr int LPR = SG::LPR, RPI = SG::RPI, NKI = SG::NKI;
    constexpr int LPT = SG::LPT, TPI = SG::TPI, NVI = SG::NVI;
    constexpr int ES = SG::ES;
    constexpr bool DQK = SG::DQK, DV = SG::DV;
    constexpr int NSC = 8;  // scalar ring depth (chunk mod 8)

    // LDS (ring slots by chunk mod NR, the scalars by chunk mod NSC, exchanges by parity):
    //   s_k   K rows of a chunk (NS bf16 planes, swizzled granules)
    //   s_q   Q rows of a chunk (as s_k)
    //   s_pt  Ptil^T, s_h H, s_tf T' of a chunk (fragments, hi and lo pieces)
    //   s_v   the V block of a chunk: bf16 rows, or channel-major fp32
    //   s_sc  the scalars of a chunk (a, s, o, Gamma_C as laid out in the workspace)
    //   s_p   each state wave's part of Gamma_c P_{c+1}, by parity of c + 1
    //   s_wf  W as B fragments (hi, lo), s_uf U (fp32, accumulator layout), by parity
    //   s_qm  each state wave's part of (Q M)^T for a chunk's outputs, by parity
    __shared__ __align__(16) char s_k[NR][SG::K_BYTES];
    __shared__ __align__(16) char s_q[SG::NRQ][SG::Q_BYTES];
    __shared__ __align__(16) bf16x8 s_pt[NR][2 * NTRI][64];
    __shared__ __align__(16) bf16x8 s_h[NR][2 * NHF][64];
    __shared__ __align__(16) bf16x8 s_tf[NR][2 * NTRI][64];
    __shared__ __align__(16) char s_v[NR][SG::V_BYTES];
    __shared__ __align__(16) float s_sc[NSC][256];
    __shared__ __align__(16) floatx4 s_p[2][NSW][RT][64];
    __shared__ __align__(16) bf16x8 s_wf[2][KTC][2][64];
    __shared__ __align__(16) floatx4 s_uf[2][RT][64];
    __shared__ __align__(16) floatx4 s_qm[2][NSW][RT][64];

    // Workgroups that share a QK head run on the same XCD (blockIdx % 8 picks the XCD), so
    // their common K/Q/H/T'/Ptil reads meet in one L2.
    int64_t lin = blockIdx.x;
    if (nblocks % 8 == 0) lin = (int64_t)(blockIdx.x % 8) * (nblocks / 8) + blockIdx.x / 8;
    const int cb = (int)(lin % (D / 16));
    const int64_t nh = lin / (D / 16);
    const int64_t seq = nh / h_v;
    const int h = (int)(nh - seq * h_v);
    const int hq = h / (h_v / h_qk);
    const int tid = threadIdx.x, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
    const int64_t nch = L.nch;
    const int64_t cend = -2 + ((nch + 3) & ~(int64_t)1);  // windows -2 .. cend - 1, an even count

    // Byte strides between consecutive tokens of q/k, v and out.
    const int64_t row_qk = (int64_t)h_qk * D * ES;
    const int64_t row_v = (int64_t)h_v * D * ES;
    const int64_t row_o = (int64_t)h_v * D * 4;
    auto par = [](int64_t c) { return (int)(c & 1); };
    auto ring = [](int64_t c) { return (int)(c % NR); };  // c >= 0
    auto qslot = [](int64_t c) { return (int)(c % SG::NRQ); };
    auto clampc = [&](int64_t c) { return c < 0 ? 0 : (c < nch ? c : nch - 1); };
    auto tok0_of = [&](int64_t c) { return seq * T + c * C; };
    auto rows_of = [&](int64_t c) { return (T - c * C) < C ? (T - c * C) : (int64_t)C; };
    auto vh_of = [&](int64_t c) { return (size_t)((seq * nch + c) * h_v + h); };
    auto sc_rsrc = [&](int64_t c) { return make_rsrc(ws + L.sc + vh_of(c) * G::SC_BYTES, G::SC_BYTES); };
    auto ws_rsrc = [&](size_t region, size_t bytes, int64_t c) {
        return make_rsrc(ws + region + vh_of(c) * bytes, (int64_t)bytes);
    };
    // q or k rows of chunk c (rows past the sequence read zero)
    auto qk_rsrc = [&](const TIn* base, int64_t c) {
        return make_rsrc(base + (tok0_of(c) * h_qk + hq) * (int64_t)D, (rows_of(c) - 1) * row_qk + D * ES);
    };
    // A lane-dependent condition selects between two constants and is added, rather than
    // guarding the address computation: lane-divergent branches anywhere in this kernel
    // would let the register allocator place copies under a partial exec mask.
    auto pad_if = [&](bool in_range) { return in_range ? 0u : OOR; };
    // Byte offset of granule j of staged row r.
    auto srow = [&](int r, int j) { return r * ROWB + 16 * (j ^ swz<RPB>(r)); };
    // A full wait: nothing left in flight, so the compiler's wait bookkeeping starts clean.
    auto settle = [&]() { __builtin_amdgcn_s_waitcnt(0); };
    // Four consecutive staged values of accumulator rows 4 lg .. 4 lg + 3 of row tile rt.
    auto sc4 = [&](int64_t c, int off) { return *reinterpret_cast<const floatx4*>(&s_sc[c & (NSC - 1)][off + 4 * lg]); };
    auto gc_of = [&](int64_t c) { return s_sc[c & (NSC - 1)][3 * CP]; };
    // V of tokens 16 rt + 4 lg + 0..3, channel lr (bf16 rows: one transposing read in which
    // lane 4 p + q of each 16-lane group addresses token 16 rt + 4 lg + p, channels 4 q ..)
    using VRaw = typename std::conditional<DV, bf16x4, floatx4>::type;
    auto vt4 = [&](int64_t c, int rt) -> VRaw {
        const char* base = s_v[ring(c)];
        if constexpr (DV)
            return lds_read_tr16(base + (16 * rt + 4 * lg + (lr >> 2)) * 32 + 8 * (lr & 3));
        else
            return *reinterpret_cast<const floatx4*>(base + (lr * SG::VS + 16 * rt + 4 * lg) * 4);
    };
    auto vf4 = [](const VRaw& x) {
        if constexpr (DV) return floatx4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
        else return x;
    };
    // Cache-line touches: one 128-byte line per lane of a chunk's inputs (its K and Q rows
    // go round the workgroups of the QK head, its workspace blocks and V rows round the
    // workgroups of the V head; lanes past this workgroup's share touch lane 0's line), so
    // that the staging loads of the chunk find the lines in L2 rather than all waiting on the
    // same misses. A lane's line moves by a fixed stride from chunk to chunk: touch_base and
    // touch_step are its address in chunk 0 and that stride (for full chunks; a partial last
    // chunk is touched as the chunk before it, or not at all when it is the only one).
    // Lane-dependent choices blend precomputed values with masks (no branches).
    uint64_t touch_base, touch_step;
    {
        constexpr int LPR128 = (D * ES + 127) / 128;  // cache lines per q/k/v row
        constexpr int NCB = D / 16;
        constexpr int TL = (int)(G::TRI_BYTES / 128), HL = (int)(G::H_BYTES / 128);
        constexpr int SCL = (int)((G::SC_BYTES + 127) / 128) - 1;  // lines starting inside
        constexpr int NWS = 2 * TL + HL + SCL;
        constexpr int HALF = C * LPR128;
        auto pick = [](bool cond, uint64_t x, uint64_t y) {
            const uint64_t m = 0 - (uint64_t)cond;
            return (x & m) | (y & ~m);
        };
        const int grp = h_v / h_qk, nbq = grp * NCB, iq = (h % grp) * NCB + cb;
        const int nq_mine = (2 * HALF - iq + nbq - 1) / nbq;
        const int nv_mine = (NWS + HALF - cb + NCB - 1) / NCB;
        const int li = l < nq_mine + nv_mine ? l : 0;
        const bool isq = li < nq_mine;
        const int lq = iq + nbq * li, rq = lq < HALF ? lq : lq - HALF;
        const uint64_t q0 = pick(lq < HALF, (uint64_t)k, (uint64_t)q) +
                            (uint64_t)(((seq * T + rq / LPR128) * h_qk + hq) * (int64_t)D * ES + 128 * (rq % LPR128));
        const uint64_t qs = (uint64_t)C * h_qk * D * ES;
        const int lv = isq ? 0 : cb + NCB * (li - nq_mine);
        const uint64_t vh0 = (uint64_t)(seq * nch * h_v + h), wsb = (uint64_t)ws;
        const uint64_t w_tt = wsb + L.tt + vh0 * G::TRI_BYTES + 128 * lv;
        const uint64_t w_pt = wsb + L.pt + vh0 * G::TRI_BYTES + 128 * (lv - TL);
        const uint64_t w_hh = wsb + L.hh + vh0 * G::H_BYTES + 128 * (lv - 2 * TL);
        const uint64_t w_sc = wsb + L.sc + vh0 * G::SC_BYTES + 128 * (lv - 2 * TL - HL);
        uint64_t w0 = pick(lv < 2 * TL + HL, w_hh, w_sc);
        uint64_t ws_step = pick(lv < 2 * TL + HL, (uint64_t)h_v * G::H_BYTES, (uint64_t)h_v * G::SC_BYTES);
        w0 = pick(lv < 2 * TL, w_pt, w0);
        w0 = pick(lv < TL, w_tt, w0);
        ws_step = pick(lv < 2 * TL, (uint64_t)h_v * G::TRI_BYTES, ws_step);
        const int rv = lv - NWS;
        const uint64_t v0 = (uint64_t)v + (uint64_t)(((seq * T + rv / LPR128) * h_v + h) * (int64_t)D * ES + 128 * (rv % LPR128));
        const uint64_t vs = (uint64_t)C * h_v * D * ES;
        touch_base = pick(isq, q0, pick(lv < NWS, w0, v0));
        touch_step = pick(isq, qs, pick(lv < NWS, ws_step, vs));
    }
    auto touch_ptr = [&](int64_t j) -> const uint32_t* {
        const int64_t jj = rows_of(j) == C ? j : j - 1;
        return reinterpret_cast<const uint32_t*>(jj >= 0 ? touch_base + (uint64_t)jj * touch_step : (uint64_t)ws);
    };

    if (w == 0) {
        // ======================================================= chain wave
        // Window c forms X_{c+1}, U_{c+1}, W_{c+1} from inputs read in window c - 1 (V, a, s
        // and T' of chunk c + 1) and from H_c X_c, formed in window c - 1 as soon as X_c was
        // known; so after the barrier only the state waves' partials are awaited.
        struct CIn { VRaw v[RT]; floatx4 a[RT], s[RT]; bf16x8 tf[2 * NTRI]; };
        auto fetch = [&](CIn& x, int64_t j) {  // inputs of chunk j
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                x.v[rt] = vt4(j, rt);
                x.a[rt] = sc4(j, 16 * rt);
                x.s[rt] = sc4(j, CP + 16 * rt);
            }
#pragma unroll
            for (int pi = 0; pi < 2 * NTRI; ++pi) x.tf[pi] = s_tf[ring(j)][pi][l];
        };
        __syncthreads();  // the staged-row buffers are cleared and the first inputs staged
        bf16x8 xf[KTC][2];  // X of the latest chunk as B fragments (hi, lo)
        floatx4 hx[RT];     // H_c X_c for the next window
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) hx[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
        // A window has no branches, so that the compiler keeps every LDS read right after the
        // barrier: slots of chunks that do not exist are read too (any contents do), and their
        // products land in exchange buffers that nobody reads. X of such a window is set to
        // zero, which keeps H X of the first window zero.
        auto window = [&](int64_t c, const CIn& cur, CIn& nxt, uint32_t& touched) {
            __syncthreads();
            const int pn = par(c + 1);
            floatx4 z[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                z[rt] = s_p[pn][0][rt][l];
#pragma unroll
                for (int sw = 1; sw < NSW; ++sw) z[rt] += s_p[pn][sw][rt][l];
            }
            const int hs = ring(c + 1 < 0 ? 0 : c + 1);
            bf16x8 hf[RT][KTC][2];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kt = 0; kt < KTC; ++kt)
#pragma unroll
                    for (int p = 0; p < 2; ++p) hf[rt][kt][p] = s_h[hs][2 * (rt * KTC + kt) + p][l];
            fetch(nxt, c + 2 < 0 ? 0 : c + 2);
            const bool live = c >= -1 && c + 1 < nch;  // wave-uniform
            // X_{c+1} = V - diag(a) (Gamma_c P_{c+1} + H_c X_c)
            floatx4 xv[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const floatx4 x = vf4(cur.v[rt]) - cur.a[rt] * (z[rt] + hx[rt]);
#pragma unroll
                for (int e = 0; e < 4; ++e) xv[rt][e] = live ? x[e] : 0.f;
            }
            rows_to_frags<RT, KTC>(xv, xf);
            // U = T' X (lower triangular: row tile rt uses token k tiles 0 .. rt / 2)
            floatx4 u[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; 2 * kt <= rt; ++kt) {
                    const int pi = 2 * (tri_off(rt) + kt);
                    acc = mfma_split<2, 2>(&cur.tf[pi], xf[kt], acc);
                }
                u[rt] = acc;
            }
            // H_{c+1} X_{c+1} for the next window
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; kt < KTC; ++kt) acc = mfma_split<2, 2>(hf[rt][kt], xf[kt], acc);
                hx[rt] = acc;
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) s_uf[pn][rt][l] = u[rt];
            // W = diag(s) U for the state waves
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) u[rt] *= cur.s[rt];
            bf16x8 wf[KTC][2];
            rows_to_frags<RT, KTC>(u, wf);
#pragma unroll
            for (int kt = 0; kt < KTC; ++kt)
#pragma unroll
                for (int p = 0; p < 2; ++p) s_wf[pn][kt][p][l] = wf[kt][p];
            // Touch the cache lines of chunk c + 8 (the staging loads of a chunk start four
            // windows before its use), after waiting for the touch of window c - 2: this wave
            // issues no other vector memory operations, so the wait counts exactly.
            asm volatile("" ::"v"(touched));
            touched = *(const __attribute__((address_space(1))) uint32_t*)touch_ptr(clampc(c + 8));
        };
        // Chunk parity alternates between windows, and so do the two input sets: window c
        // uses the set of chunk c + 1 and fills that of chunk c + 2.
        CIn A, B;
        uint32_t ta = 0, tb = 0;
#pragma unroll 1
        for (int64_t c = -2; c < cend; c += 2) {
            window(c, B, A, ta);
            window(c + 1, A, B, tb);
        }
    } else if (w <= NSW) {
        // ======================================================= state wave sw
        // State tiles 2 KPS sw .. 2 KPS (sw + 1) - 1, i.e. d_k tiles KPS sw .. KPS (sw + 1) - 1.
        const int sw = w - 1;
        const int64_t sbase = nh * (int64_t)D * D;
        // The state block through buffer resources: padded features (D = 16) fall outside
        // the range, and a missing initial state is an empty range, so both read zero.
        auto st_off = [&](int mt, int e) {
            const int f = feat_of(mt, 4 * lg + e);
            return (int)((uint32_t)((f * D + cb * 16 + lr) * 4) + pad_if(f < D));
        };
        floatx4 macc[2 * KPS];
        {
            const auto r = make_rsrc(state_in + (state_in ? sbase : 0), state_in ? (int64_t)D * D * 4 : 0);
#pragma unroll
            for (int i = 0; i < 2 * KPS; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) macc[i][e] = buf_elem<float>(r, st_off(2 * KPS * sw + i, e));
        }
        bf16x8 mf[KPS][2];  // this wave's d_k tiles of the state as B fragments (hi, lo)
        auto split = [&]() {
#pragma unroll
            for (int kk = 0; kk < KPS; ++kk) pair_to_frag(macc[2 * kk], macc[2 * kk + 1], mf[kk][0], mf[kk][1]);
        };
        split();          // the state entering chunk 0
        __syncthreads();  // the staged-row buffers are cleared and the first inputs staged
        // A fragment pieces of staged rows (K or Q of a chunk): rows 16 rt + 0..15, the features
        // of this wave's d_k tile kk.
        auto row_frag = [&](const char* rows, int rt, int kk, bf16x8* a) {
#pragma unroll
            for (int part = 0; part < NS; ++part)
                a[part] = *reinterpret_cast<const bf16x8*>(
                    rows + part * CP * ROWB + srow(16 * rt + lr, 4 * (KPS * sw + kk) + lg));
        };

        // K^T A fragments of a chunk for this wave's state tiles, read two windows before the
        // state update that uses them (when the chunk's rows are first used for P; the ring
        // slot is refilled before the update). Fragment (i, kt): two transposing reads (token slots
        // 0..3, 4..7); lane lr of group lg addresses token row 32 kt + 16 h + 4 lg + lr / 4 and
        // features 32 (KPS sw + i / 2) + 8 (lr % 4) + 4 (i % 2) + 0..3.
        bf16x8 ktA[2 * KPS][KTC][NS], ktB[2 * KPS][KTC][NS];
#pragma unroll
        for (int i = 0; i < 2 * KPS; ++i)
#pragma unroll
            for (int kt = 0; kt < KTC; ++kt)
#pragma unroll
                for (int part = 0; part < NS; ++part) ktA[i][kt][part] = ktB[i][kt][part] = bf16x8{};
        auto read_kt = [&](bf16x8 (*kts)[KTC][NS], int slot) {
#pragma unroll
            for (int i = 0; i < 2 * KPS; ++i)
#pragma unroll
                for (int kt = 0; kt < KTC; ++kt)
#pragma unroll
                    for (int part = 0; part < NS; ++part) {
                        const int r = 32 * kt + 4 * lg + (lr >> 2);
                        const int j = 4 * (KPS * sw + (i >> 1)) + (lr & 3);
                        const char* base = s_k[slot] + part * CP * ROWB + 8 * (i & 1);
                        const bf16x4 a = lds_read_tr16(base + srow(r, j));
                        const bf16x4 b = lds_read_tr16(base + srow(r + 16, j));
                        kts[i][kt][part] = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
                    }
        };
        // Every LDS read of a window is issued right after its barrier, so that the state
        // update, the split and the products wait for one round of reads; the window has no
        // branches, so the compiler keeps the reads there. Slots are read even when their
        // chunk does not exist (any contents do), and the products of such windows land in
        // exchange buffers nobody reads. Without a chunk the update is M <- 1 * M + K^T 0,
        // exact, with W selected to zero and K^T finite (staged rows or zero).
        auto window = [&](int64_t c, bf16x8 (*kts)[KTC][NS]) {
            __syncthreads();
            const int64_t c1 = c + 1 < 0 ? 0 : c + 1, c2 = c + 2 < 0 ? 0 : c + 2;
            bf16x8 wf[KTC][2];
#pragma unroll
            for (int kt = 0; kt < KTC; ++kt)
#pragma unroll
                for (int p = 0; p < 2; ++p) wf[kt][p] = s_wf[par(c)][kt][p][l];
            bf16x8 qa[RT][KPS][NS], ka[RT][KPS][NS];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kk = 0; kk < KPS; ++kk) {
                    row_frag(s_q[qslot(c1)], rt, kk, qa[rt][kk]);
                    row_frag(s_k[ring(c2)], rt, kk, ka[rt][kk]);
                }
            const bool upd = c >= 0 && c < nch;  // wave-uniform
            const float gcc = upd ? gc_of(c) : 1.f, gc1 = gc_of(c1);
#pragma unroll
            for (int kt = 0; kt < KTC; ++kt)
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    u32x4 x = __builtin_bit_cast(u32x4, wf[kt][p]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = upd ? x[e] : 0u;
                    wf[kt][p] = __builtin_bit_cast(bf16x8, x);
                }
            // M_{c+1} = Gamma_c M_c + K_c^T W_c
#pragma unroll
            for (int i = 0; i < 2 * KPS; ++i) {
                floatx4 acc = gcc * macc[i];
#pragma unroll
                for (int kt = 0; kt < KTC; ++kt) acc = mfma_split<NS, 2>(kts[i][kt], wf[kt], acc);
                macc[i] = acc;
            }
            // K^T of chunk c + 2 replaces K^T of chunk c as soon as the update has issued, so
            // the reads overlap the split and the products below.
            read_kt(kts, ring(c2));
            split();  // the state entering chunk c + 1
            // (Q_{c+1} M_{c+1})^T over this wave's features, for the output helpers: the state
            // fragments serve as A operands and the Q row fragments as B operands, so each lane
            // ends up with four value channels of one token
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KPS; ++kk) acc = mfma_split<2, NS>(mf[kk], qa[rt][kk], acc);
                s_qm[par(c1)][sw][rt][l] = acc;
            }
            // Gamma_{c+1} K_{c+2} M_{c+1} over this wave's features (unscaled for chunk 0)
            const float scale = c >= -1 ? gc1 : 1.f;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KPS; ++kk) acc = mfma_split<NS, 2>(ka[rt][kk], mf[kk], acc);
                s_p[par(c2)][sw][rt][l] = scale * acc;
            }
        };
        // Chunk parity alternates between windows, and so do the two K^T register sets.
#pragma unroll 1
        for (int64_t c = -2; c < cend; c += 2) {
            window(c, ktA);
            window(c + 1, ktB);
        }

        {
            const auto r = make_rsrc(state_out + sbase, (int64_t)D * D * 4);
#pragma unroll
            for (int i = 0; i < 2 * KPS; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float val = macc[i][e];
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), r, st_off(2 * KPS * sw + i, e), 0, 0);
                }
        }
    } else {
        // ======================================================= helper wave hw
        // Helpers 0 .. NOH - 1 form the outputs of row tile hw; the others stage the inputs.
        // Each helper runs code specialised for its index, so its sequence of vector memory
        // operations has no branches and the waits below count exactly.
        const int hw = w - 1 - NSW;

        // Clear the staged rows once: rows past a short chunk and features past D are never
        // written afterwards and must read as zero. (The size is a multiple of 1 KB, so every
        // lane makes the same number of trips.)
        for (int o = 1024 * hw; o < (int)(NR * SG::K_BYTES); o += 1024 * NHW)
            *reinterpret_cast<u32x4*>(&s_k[0][0] + o + 16 * l) = u32x4{0u, 0u, 0u, 0u};
        for (int o = 1024 * hw; o < (int)(SG::NRQ * SG::Q_BYTES); o += 1024 * NHW)
            *reinterpret_cast<u32x4*>(&s_q[0][0] + o + 16 * l) = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();

        auto output_helper = [&](auto hw_const) {
            constexpr int RTO = decltype(hw_const)::value;  // the row tile of this helper
            // Outputs of chunk c, formed transposed: O^T = (Q M_c)^T diag(o) + U^T Ptil^T as 16
            // value channels x 16 tokens tiles. The state waves' parts of (Q M_c)^T are summed;
            // the U fragments serve as A operands and Ptil^T as B operands, and each lane ends
            // up with four consecutive channels of one token (one 16-byte store). Windows
            // outside the chunks store out of range.
            auto do_output = [&](int64_t c) {
                const bool live = c >= 0 && c < nch;  // wave-uniform
                c = clampc(c);
                const int pc = par(c), slot = ring(c);
                floatx4 urow[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) urow[rt] = s_uf[pc][rt][l];
                floatx4 qm = s_qm[pc][0][RTO][l];
#pragma unroll
                for (int sw = 1; sw < NSW; ++sw) qm += s_qm[pc][sw][RTO][l];
                const float o = s_sc[c & (NSC - 1)][2 * CP + 16 * RTO + lr];  // o of token 16 RTO + lr
                bf16x8 ufr[KTC][2];
                rows_to_frags<RT, KTC>(urow, ufr);
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; 2 * kt <= RTO; ++kt) {
                    const int pi = 2 * (tri_off(RTO) + kt);
                    const bf16x8 pf[2] = {s_pt[slot][pi][l], s_pt[slot][pi + 1][l]};
                    acc = mfma_split<2, 2>(ufr[kt], pf, acc);
                }
                acc += o * qm;
                const auto r_o = make_rsrc(out + (tok0_of(c) * h_v + h) * (int64_t)D + cb * 16,
                                           (rows_of(c) - 1) * row_o + 64);
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4, acc), r_o,
                    (int)((uint32_t)((16 * RTO + lr) * row_o) + (uint32_t)(lg * 16) + pad_if(live)), 0, 0);
            };
#pragma unroll 1
            for (int64_t c = -2; c < cend; ++c) {
                __syncthreads();
                do_output(c);
            }
            settle();
        };

        auto staging_helper = [&](auto hs_const) {
            constexpr int HS = decltype(hs_const)::value;  // index among the staging helpers
            // This helper's shares: loads m of it cover items HS + NSH m.
            constexpr auto share = [](int n) { return n > HS ? (n - HS + NSH - 1) / NSH : 0; };
            constexpr int NKM = share(NKI);                       // K (and Q) row loads
            constexpr int NTM = share(2 * NTRI), NHM = share(2 * NHF), NPM = share(2 * NTRI);
            constexpr bool VST = HS == NSH - 1;                   // the V block and the scalars
            // Register-staged inputs (fp32 or d = 16 K and Q rows; fp32 V): the set of window c
            // holds the K rows and the V block of chunk c + 3 and the Q rows of chunk c + 2,
            // loaded two windows earlier; two sets alternate.
            constexpr bool RK = !DQK, RV = !DV && VST;
            struct RSet {
                u32x4 kr[RK && NKM > 0 ? NKM : 1];
                u32x4 qr[RK && NKM > 0 ? NKM : 1];
                u32x4 vr[RV ? NVI : 1];
            };
            // K or Q rows of chunk c straight into ring slot `dst`: load m covers rows
            // RPI (HS + NSH m) .., whose staged bytes form 1 KB; lane l lands at position l of it.
            auto dma_rows = [&](const TIn* base, int64_t c, char* dst) {
                const auto r = qk_rsrc(base, clampc(c));
#pragma unroll
                for (int m = 0; m < NKM; ++m) {
                    const int mi = HS + NSH * m;
                    const int row = RPI * mi + l / NG, pos = l % NG;
                    const int g = pos ^ swz<RPB>(row);
                    load_to_lds(r, dst + mi * 1024,
                                (int)((uint32_t)(row * row_qk) + (uint32_t)(16 * g) + pad_if(row < C)));
                }
            };
            // Fragment pieces HS + NSH m (1 KB each) of a workspace block into `dst`.
            auto dma_pieces = [&](size_t region, size_t bytes, int64_t c, bf16x8 (*dst)[64], int n) {
                const auto r = ws_rsrc(region, bytes, clampc(c));
#pragma unroll
                for (int m = 0; HS + NSH * m < n; ++m)
                    load_to_lds(r, dst[HS + NSH * m], (HS + NSH * m) * 1024 + l * 16);
            };
            auto ld_rows = [&](const TIn* base, int64_t c, u32x4* dst) {
                const auto r = qk_rsrc(base, clampc(c));
#pragma unroll
                for (int m = 0; m < NKM; ++m) {
                    const int row = RPI * (HS + NSH * m) + l / LPR;
                    dst[m] = __builtin_amdgcn_raw_buffer_load_b128(
                        r, (int)((uint32_t)(row * row_qk) + (uint32_t)(16 * (l % LPR)) + pad_if(row < C)), 0, 0);
                }
            };
            auto ld_regs = [&](RSet& x, int64_t c) {  // the set of window c
                if constexpr (RK) {
                    ld_rows(k, c + 3, x.kr);
                    ld_rows(q, c + 2, x.qr);
                }
                if constexpr (RV) {
                    const int64_t c3 = clampc(c + 3);
                    const auto r_v = make_rsrc(v + (tok0_of(c3) * h_v + h) * (int64_t)D + cb * 16,
                                               (rows_of(c3) - 1) * row_v + 16 * ES);
#pragma unroll
                    for (int m = 0; m < NVI; ++m) {
                        const int t = TPI * m + l / LPT;
                        x.vr[m] = __builtin_amdgcn_raw_buffer_load_b128(
                            r_v, (int)((uint32_t)(t * row_v) + (uint32_t)(16 * (l % LPT)) + pad_if(t < C)), 0, 0);
                    }
                }
            };
            // Register-loaded rows into staged rows (fp32 split into hi and lo planes).
            auto st_rows = [&](const u32x4* src, char* dst) {
#pragma unroll
                for (int m = 0; m < NKM; ++m) {
                    const int row = RPI * (HS + NSH * m) + l / LPR, g = l % LPR;
                    if constexpr (ES == 2) {
                        *reinterpret_cast<u32x4*>(dst + srow(row, g)) = src[m];
                    } else {
                        const floatx4 y = __builtin_bit_cast(floatx4, src[m]);
                        uint32_t hi[2], lo[2];
                        split2(y[0], y[1], &hi[0], &lo[0]);
                        split2(y[2], y[3], &hi[1], &lo[1]);
                        const int o = srow(row, g >> 1) + 8 * (g & 1);
                        *reinterpret_cast<uint2*>(dst + o) = uint2{hi[0], hi[1]};
                        *reinterpret_cast<uint2*>(dst + CP * ROWB + o) = uint2{lo[0], lo[1]};
                    }
                }
            };
            // The register-staged inputs of window c (K and V of chunk c + 3, Q of chunk c + 2).
            auto st_regs = [&](const RSet& x, int64_t c) {
                if constexpr (RK) {
                    if (c + 3 >= 0 && c + 3 < nch) st_rows(x.kr, s_k[ring(c + 3)]);
                    if (c + 2 >= 0 && c + 2 < nch) st_rows(x.qr, s_q[qslot(c + 2)]);
                }
                if constexpr (RV) {
                    if (c + 3 >= 0 && c + 3 < nch) {
                        float* dst = reinterpret_cast<float*>(s_v[ring(c + 3)]);
#pragma unroll
                        for (int m = 0; m < NVI; ++m) {
                            const int t = TPI * m + l / LPT;  // < CP
                            const floatx4 y = __builtin_bit_cast(floatx4, x.vr[m]);
#pragma unroll
                            for (int e = 0; e < 4; ++e) dst[(4 * (l % LPT) + e) * SG::VS + t] = y[e];
                        }
                    }
                }
            };
            // The loads straight into LDS issued in window c (clamped chunks beyond the
            // sequence land in ring slots nobody reads any more).
            // The chain's inputs of chunk j (T', the V block, the scalars).
            auto dma_chain = [&](int64_t j) {
                dma_pieces(L.tt, G::TRI_BYTES, j, s_tf[ring(j)], 2 * NTRI);
                if constexpr (VST) {
                    const int64_t jc = clampc(j);
                    if constexpr (DV) {
                        const auto r_v = make_rsrc(v + (tok0_of(jc) * h_v + h) * (int64_t)D + cb * 16,
                                                   (rows_of(jc) - 1) * row_v + 32);
#pragma unroll
                        for (int m = 0; m < NVI; ++m) {
                            const int t = TPI * m + l / 2;
                            load_to_lds(r_v, s_v[ring(j)] + m * 1024,
                                        (int)((uint32_t)(t * row_v) + (uint32_t)(16 * (l & 1)) + pad_if(t < C)));
                        }
                    }
                    load_to_lds(sc_rsrc(jc), s_sc[j & (NSC - 1)], 16 * l);
                }
            };
            auto issue = [&](int64_t c) {
                if constexpr (DQK) dma_rows(k, c + 4, s_k[ring(c + 4)]);
                dma_chain(c + 4);
                dma_pieces(L.hh, G::H_BYTES, c + 3, s_h[ring(c + 3)], 2 * NHF);
                if constexpr (DQK) dma_rows(q, c + 3, s_q[qslot(c + 3)]);
                dma_pieces(L.pt, G::TRI_BYTES, c + 2, s_pt[ring(c + 2)], 2 * NTRI);
            };
            // Vector memory operations one window issues: the loads straight into LDS, then
            // the register loads. Loads complete in order, so the straight loads of window c - 1
            // have landed once no more than those issued after them (the register loads of
            // windows c - 1 and c and the straight loads of window c) are in flight.
            constexpr int NDMA = (DQK ? 2 * NKM : 0) + NTM + NHM + NPM + (VST ? (DV ? NVI : 0) + 1 : 0);
            constexpr int NREG = (RK ? 2 * NKM : 0) + (RV ? NVI : 0);
            constexpr int NVM = NDMA + 2 * NREG;

            // Prologue: K rows of chunk 0 (and of chunk 1 and Q rows of chunk 0 when they load
            // straight into LDS), the chain's inputs of chunks 0 and 1 and H_0 in place; window
            // -2 writes the register-staged K rows and V block of chunk 1 and Q rows of chunk 0.
            {
                if constexpr (DQK) {
                    dma_rows(k, 0, s_k[ring(0)]);
                    dma_rows(k, 1, s_k[ring(1)]);
                    dma_rows(q, 0, s_q[qslot(0)]);
                } else {
                    RSet x0;
                    ld_regs(x0, -3);  // K rows and V block of chunk 0
                    settle();
                    st_regs(x0, -3);
                }
                dma_chain(0);
                dma_chain(1);
                dma_pieces(L.hh, G::H_BYTES, 0, s_h[ring(0)], 2 * NHF);
                settle();
            }
            RSet A, B;
            ld_regs(A, -2);
            ld_regs(B, -1);
            auto window = [&](RSet& x, int64_t c) {
                barrier_lds_only();
                st_regs(x, c);
                issue(c);
                __builtin_amdgcn_sched_barrier(0);
                ld_regs(x, c + 2);
                wait_vm<NVM>();  // the loads straight into LDS issued in window c - 1 have landed
            };
#pragma unroll 1
            for (int64_t c = -2; c < cend; c += 2) {
                window(A, c);
                window(B, c + 1);
            }
            settle();
        };

        static_assert(NOH >= 1 && NSH >= 1, "helper roles");
        // Output helpers come first and last, staging helpers in between: wave w runs on SIMD
        // w mod 4, so with two output helpers they share one SIMD and each staging helper
        // shares one with the chain or a state wave.
        dispatch_index<0, NHW>(hw, [&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i == 0) output_helper(std::integral_constant<int, 0>{});
            // (the row tile is written as a function of i, 1 here, so that the call is only
            // instantiated where the branch is taken)
            else if constexpr (NOH == 2 && i == NHW - 1)
                output_helper(std::integral_constant<int, i + 2 - NHW>{});
            else staging_helper(std::integral_constant<int, i - 1>{});
        });
    }
}

// ============================================================ scan, chunks of 64 and 128 tokens
// For longer chunks the pipeline above does not fit LDS (its staging rings and exchange
// buffers grow with the chunk). This variant keeps the state in two "chain" waves (halves of
// d_k), which run the recurrence with one exchange of partial K M0 products per chunk, while
// two "output" waves stage T', V and the scalars and form the outputs one chunk behind.
template <int D, int C, typename TIn>
struct WideGeo {
    using G = Geo<D, C, std::is_same<TIn, float>::value>;
    // Two operand sets alternate (the next chunk's loads fly while this chunk computes)
    // when both fit the register file; at C = 128 one set is loaded per chunk.
    static constexpr bool DB = C <= 64;
    // The output waves stage what both chain waves read into LDS, one chunk ahead: the T'
    // tiles (2 NTRI pieces of 1 KB, NTS per output wave) and, from the last output wave,
    // the V block (transposed to channel-major fp32) and the scalars a, s and Gamma_C.
    static constexpr int CPV = G::CP < 64 ? 64 : G::CP;  // staged token slots
    static constexpr int TPL = CPV / 64;                  // staged tokens per lane
    static constexpr int VS = CPV + 4;                    // LDS row stride of the V block
    // Each chain wave keeps the K rows of its feature half (as bf16 pieces) in LDS, where
    // transposing reads turn them into the K^T operand of the state update.
    static constexpr int KS = 32 * G::KTH + 8;            // LDS row stride of those rows
    static constexpr size_t KB_BYTES = (size_t)G::NCH * G::NS * G::CP * KS * 2;
    // LDS besides the T' tiles; where the tiles do not fit next to it (C = 128 with
    // d >= 64) the chain waves read T' from the workspace instead.
    static constexpr size_t LDS_REST = (size_t)2 * G::NCH * G::RT * 1024 + (size_t)2 * G::KTD * 2048 +
                                       (size_t)2 * G::RT * 1024 + (size_t)2 * 16 * VS * 4 +
                                       (size_t)2 * 2 * CPV * 4 + 16 + KB_BYTES;
    static constexpr bool TLDS = LDS_REST + (size_t)2 * 2 * G::NTRI * 1024 <= 160 * 1024;
    static constexpr int NTS = TLDS ? (2 * G::NTRI + G::NOW - 1) / G::NOW : 1;
};

// Operands a chain wave loads for chunk c: the K rows of chunk c + 1.
template <int D, int C, typename TIn>
struct WideChainSet {
    using G = Geo<D, C, std::is_same<TIn, float>::value>;
    typename RawFrag<TIn>::type kr[G::RT][G::KTH];  // K rows of chunk c + 1 (A fragments)
};

// Operands an output wave loads for window j (finishing chunk j - 1, starting chunk j),
// and what it stages for the chain waves' chunk j + 1.
template <int D, int C, typename TIn>
struct WideOutSet {
    using G = Geo<D, C, std::is_same<TIn, float>::value>;
    using SG = WideGeo<D, C, TIn>;
    typename RawFrag<TIn>::type qr[G::RTO][G::KTD];  // Q rows of chunk j (A fragments)
    bf16x8 pf[G::RTO][G::KTC][2];                     // Ptil^T of chunk j - 1 (B fragments)
    float ov[G::RTO];                                 // scalar o of token lr of each row tile
    bf16x8 tst[SG::NTS];                              // T' pieces of chunk j + 1
    typename RawFrag<TIn>::type vr[SG::TPL][2];      // V rows of chunk j + 1 (16 channels)
    float sa[SG::TPL], ss[SG::TPL], gc;               // a, s of those tokens; Gamma_C
};

__device__ __forceinline__ float elem_f32(const bf16x8& r, int e)
{
    return (float)r[e];
}

__device__ __forceinline__ float elem_f32(const floatx8& r, int e)
{
    return r[e];
}

template <int D, int C, typename TIn>
__global__ void __launch_bounds__(256)
chunk_scan_wide_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
                  const char* __restrict__ ws, ChunkWs L, const float* state_in,
                  float* __restrict__ out, float* state_out, int64_t T, int h_qk, int h_v,
                  int64_t nblocks)
{
    constexpr bool F32IN = std::is_same<TIn, float>::value;
    using G = Geo<D, C, F32IN>;
    using SG = WideGeo<D, C, TIn>;
    using Raw = typename RawFrag<TIn>::type;
    using CS = WideChainSet<D, C, TIn>;
    using OS = WideOutSet<D, C, TIn>;
    constexpr int CP = G::CP, RT = G::RT, KTC = G::KTC, KTD = G::KTD, NS = G::NS;
    constexpr int NTRI = G::NTRI, NCH = G::NCH, KTH = G::KTH, MTH = G::MTH;
    constexpr int NOW = G::NOW, RTO = G::RTO, NTS = SG::NTS, CPV = SG::CPV, TPL = SG::TPL;
    constexpr int ES = sizeof(TIn);

    // LDS, double-buffered by chunk parity, one 16-byte value per lane per slot where a
    // wave's fragment passes to another wave unchanged:
    //   s_xp  partial K M0 of each chain wave        s_mf  the state's B fragments (hi, lo)
    //   s_uf  U (fp32, accumulator layout)           s_tf  T' tiles
    //   s_vt  V block, channel-major fp32            s_sc  scalars a, s; s_gc Gamma_C
    __shared__ __align__(16) floatx4 s_xp[2][NCH][RT][64];
    __shared__ __align__(16) bf16x8 s_mf[2][KTD][2][64];
    __shared__ __align__(16) floatx4 s_uf[2][RT][64];
    __shared__ __align__(16) bf16x8 s_tf[SG::TLDS ? 2 : 1][SG::TLDS ? 2 * NTRI : 1][64];
    __shared__ __align__(16) __bf16 s_kb[NCH][NS][CP][SG::KS];  // each chain wave's K rows
    __shared__ __align__(16) float s_vt[2][16][SG::VS];
    __shared__ __align__(16) float s_sc[2][2][CPV];
    __shared__ float s_gc[2];

    // Workgroups that share a QK head run on the same XCD (blockIdx % 8 picks the XCD), so
    // their common K/Q/T'/Ptil reads meet in one L2.
    int64_t lin = blockIdx.x;
    if (nblocks % 8 == 0) lin = (int64_t)(blockIdx.x % 8) * (nblocks / 8) + blockIdx.x / 8;
    const int cb = (int)(lin % (D / 16));
    const int64_t nh = lin / (D / 16);
    const int64_t seq = nh / h_v;
    const int h = (int)(nh - seq * h_v);
    const int hq = h / (h_v / h_qk);
    const int tid = threadIdx.x, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
    const int64_t nch = L.nch;

    // Byte strides between consecutive tokens of q/k, v and out.
    const int64_t row_qk = (int64_t)h_qk * D * ES;
    const int64_t row_v = (int64_t)h_v * D * ES;
    const int64_t row_o = (int64_t)h_v * D * 4;
    auto clampc = [&](int64_t c) { return c < 0 ? 0 : (c < nch ? c : nch - 1); };
    auto tok0_of = [&](int64_t c) { return seq * T + c * C; };
    auto rows_of = [&](int64_t c) { return (T - c * C) < C ? (T - c * C) : (int64_t)C; };
    auto vh_of = [&](int64_t c) { return (size_t)((seq * nch + c) * h_v + h); };
    auto sc_rsrc = [&](int64_t c) { return make_rsrc(ws + L.sc + vh_of(c) * G::SC_BYTES, G::SC_BYTES); };
    // K or Q rows of chunk c as A fragments: row tile rt, feature k tile kt (features past D
    // and rows past the sequence read zero).
    auto qk_rsrc = [&](const TIn* base, int64_t c) {
        return make_rsrc(base + (tok0_of(c) * h_qk + hq) * (int64_t)D, (rows_of(c) - 1) * row_qk + D * ES);
    };
    // A lane-dependent condition selects between two constants and is added, rather than
    // guarding the address computation: lane-divergent branches anywhere in this kernel
    // would let the register allocator place copies under a partial exec mask.
    auto pad_if = [&](bool in_range) { return in_range ? 0u : OOR; };
    auto qk_off = [&](int rt, int kt) {
        const int f = 32 * kt + 8 * lg;
        return (int)((uint32_t)((16 * rt + lr) * row_qk) + (uint32_t)(f * ES) + pad_if(rt < RT && f < D));
    };
    // A full wait: nothing left in flight, so the compiler's wait bookkeeping starts clean
    // at the next chunk (no loop-carried loads that would force early waits).
    auto settle = [&]() { __builtin_amdgcn_s_waitcnt(0); };
    // Four consecutive staged values of accumulator rows 4 lg .. 4 lg + 3 of row tile rt.
    auto vt4 = [&](int par, int rt) { return *reinterpret_cast<const floatx4*>(&s_vt[par][lr][16 * rt + 4 * lg]); };
    auto sc4 = [&](int par, int which, int rt) {
        return *reinterpret_cast<const floatx4*>(&s_sc[par][which][16 * rt + 4 * lg]);
    };

    if (w < NCH) {
        // ======================================================= chain wave hh
        const int hh = w;
        // The state block through buffer resources: padded features (D = 16) fall outside
        // the range, and a missing initial state is an empty range, so both read zero.
        const int64_t sbase = nh * (int64_t)D * D;
        auto st_off = [&](int mt, int e) {
            const int f = feat_of(mt, 4 * lg + e);
            return (int)((uint32_t)((f * D + cb * 16 + lr) * 4) + pad_if(f < D));
        };
        floatx4 macc[MTH];  // state tiles hh * MTH + i
        {
            const auto r = make_rsrc(state_in + (state_in ? sbase : 0), state_in ? (int64_t)D * D * 4 : 0);
#pragma unroll
            for (int i = 0; i < MTH; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) macc[i][e] = buf_elem<float>(r, st_off(hh * MTH + i, e));
        }
        bf16x8 mf[KTH][2];  // the state as B fragments (hi, lo) of this wave's d k tiles
        auto split_state = [&]() {
#pragma unroll
            for (int kk = 0; kk < KTH; ++kk) pair_to_frag(macc[2 * kk], macc[2 * kk + 1], mf[kk][0], mf[kk][1]);
        };
        auto load_k = [&](Raw (*kr)[KTH], int64_t c) {
            const auto r = qk_rsrc(k, clampc(c));
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kk = 0; kk < KTH; ++kk) kr[rt][kk] = buf_raw_frag<TIn>(r, qk_off(rt, hh * KTH + kk));
        };
        // This wave's K rows into its LDS buffer (row-major, features of its half; rows past
        // the chunk stay zero). Only this wave reads them back, after its own writes.
        auto store_k = [&](const Raw (*kr)[KTH]) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kk = 0; kk < KTH; ++kk) {
                    bf16x8 piece[NS];
                    to_pieces(kr[rt][kk], piece);
#pragma unroll
                    for (int part = 0; part < NS; ++part)
                        *reinterpret_cast<bf16x8*>(&s_kb[hh][part][16 * rt + lr][32 * kk + 8 * lg]) = piece[part];
                }
        };
        if constexpr (16 * RT < CP) {  // C = 16: token rows 16..31 of the padded k tile
            for (int i = l; i < NS * (CP - 16 * RT) * SG::KS; i += 64) {
                const int part = i / ((CP - 16 * RT) * SG::KS), rem = i % ((CP - 16 * RT) * SG::KS);
                s_kb[hh][part][16 * RT + rem / SG::KS][rem % SG::KS] = (__bf16)0.f;
            }
        }
        // K^T A fragment of this wave's state tile i, token k tile kt: two transposing reads,
        // for token slots 0..3 and 4..7 (lane lr of group lg addresses token row
        // 32 kt + 16 h + 4 lg + lr / 4 and the four features feat_of(mt, 4 (lr % 4) + 0..3)).
        auto kt_frag = [&](int i, int kt, int part) {
            const int col = 32 * (i >> 1) + 8 * (lr & 3) + 4 * (i & 1);
            const int row = 32 * kt + 4 * lg + (lr >> 2);
            const bf16x4 a = lds_read_tr16(&s_kb[hh][part][row][col]);
            const bf16x4 b = lds_read_tr16(&s_kb[hh][part][row + 16][col]);
            return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        };

        // This wave's part of K M0 for the chunk whose K rows are given.
        floatx4 pp[RT];
        auto partial_km = [&](const Raw (*kr)[KTH]) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KTH; ++kk) {
                    bf16x8 ka[NS];
                    to_pieces(kr[rt][kk], ka);
                    acc = mfma_split<NS, 2>(ka, mf[kk], acc);
                }
                pp[rt] = acc;
            }
        };
        auto publish = [&](int par) {
            if constexpr (NCH > 1) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) s_xp[par][hh][rt][l] = pp[rt];
            }
#pragma unroll
            for (int kk = 0; kk < KTH; ++kk)
#pragma unroll
                for (int p = 0; p < 2; ++p) s_mf[par][hh * KTH + kk][p][l] = mf[kk][p];
        };

        // One chunk, between the barrier that publishes its inputs and the next one. The K
        // rows are reloaded for the next chunk right after their last use here (the
        // scheduling barrier keeps the loads behind that use), so one register set
        // suffices and the loads have about a chunk to arrive.
        CS x;
        auto window = [&](int64_t c) {
            const int par = (int)(c & 1);
            // T' first: nothing in this chunk computes it, so its LDS latency overlaps X.
            bf16x8 tfr[SG::TLDS ? 2 * NTRI : 1];
            if constexpr (SG::TLDS) {
#pragma unroll
                for (int pi = 0; pi < 2 * NTRI; ++pi) tfr[pi] = s_tf[par][pi][l];
            }
            // X = V - diag(a) K M0, with K M0 the sum of both waves' parts (the same order of
            // addition in both waves, so both compute identical U)
            floatx4 xv[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                floatx4 z = pp[rt];
                if constexpr (NCH > 1) z += s_xp[par][hh ^ 1][rt][l];
                xv[rt] = vt4(par, rt) - sc4(par, 0, rt) * z;
            }
            bf16x8 xf[KTC][2];
            rows_to_frags<RT, KTC>(xv, xf);
            const auto r_t = make_rsrc(ws + L.tt + vh_of(c) * G::TRI_BYTES, SG::TLDS ? 0 : G::TRI_BYTES);
            // U = T' X (lower triangular: row tile rt uses token k tiles 0 .. rt / 2)
            floatx4 u[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; 2 * kt <= rt; ++kt) {
                    const int pi = 2 * (tri_off(rt) + kt);
                    bf16x8 tf[2];
                    if constexpr (SG::TLDS) {
                        tf[0] = tfr[pi];
                        tf[1] = tfr[pi + 1];
                    } else {
                        tf[0] = buf_bf16x8(r_t, pi * 1024 + l * 16);
                        tf[1] = buf_bf16x8(r_t, pi * 1024 + 1024 + l * 16);
                    }
                    acc = mfma_split<2, 2>(tf, xf[kt], acc);
                }
                u[rt] = acc;
            }
            if (hh == 0) {  // U for the output waves
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) s_uf[par][rt][l] = u[rt];
            }
            // W = diag(s) U;  M <- Gamma_C M + K^T W
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) u[rt] *= sc4(par, 1, rt);
            bf16x8 wf[KTC][2];
            rows_to_frags<RT, KTC>(u, wf);
            const float gc = s_gc[par];
#pragma unroll
            for (int i = 0; i < MTH; ++i) {
                floatx4 acc = gc * macc[i];
#pragma unroll
                for (int kt = 0; kt < KTC; ++kt) {
                    bf16x8 ktp[NS];
#pragma unroll
                    for (int part = 0; part < NS; ++part) ktp[part] = kt_frag(i, kt, part);
                    acc = mfma_split<NS, 2>(ktp, wf[kt], acc);
                }
                macc[i] = acc;
            }
            // The next chunk's partial K M0 (past the last chunk: computed on reloaded rows
            // and never read); its K rows replace this chunk's in LDS.
            split_state();
            partial_km(x.kr);
            store_k(x.kr);
            __builtin_amdgcn_sched_barrier(0);
            load_k(x.kr, c + 2);
            publish(par ^ 1);
        };

        split_state();
        load_k(x.kr, 0);
        partial_km(x.kr);
        store_k(x.kr);
        publish(0);
        load_k(x.kr, 1);
#pragma unroll 1
        for (int64_t c = 0; c < nch; ++c) {
            __syncthreads();
            window(c);
        }
        __syncthreads();  // matches the output waves' last window

        {
            const auto r = make_rsrc(state_out + sbase, (int64_t)D * D * 4);
#pragma unroll
            for (int i = 0; i < MTH; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float val = macc[i][e];
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), r, st_off(hh * MTH + i, e), 0, 0);
                }
        }
    } else {
        // ======================================================= output wave ow
        // Row tiles ow, ow + NOW, ...; one chunk behind the chain waves. Window j finishes
        // the outputs of chunk j - 1 and starts (Q M0)^T of chunk j.
        const int ow = w - NCH;
        const bool stager = ow == NOW - 1;  // wave-uniform
        floatx4 qm[RTO];  // (Q M0)^T of the chunk being finished

        // What the chain waves read in chunk c: T' pieces (every output wave) and the V
        // block, a, s and Gamma_C (the stager).
        auto load_stage = [&](OS& x, int64_t c) {
            c = clampc(c);
            if constexpr (SG::TLDS) {
                const auto r = make_rsrc(ws + L.tt + vh_of(c) * G::TRI_BYTES, G::TRI_BYTES);
#pragma unroll
                for (int m = 0; m < NTS; ++m) {
                    const int pi = ow + NOW * m;
                    x.tst[m] = buf_bf16x8(r, pi < 2 * NTRI ? pi * 1024 + l * 16 : (int)OOR);
                }
            }
            if (stager) {
                const auto r_v = make_rsrc(v + (tok0_of(c) * h_v + h) * (int64_t)D + cb * 16,
                                           (rows_of(c) - 1) * row_v + 16 * ES);
                const auto rs = sc_rsrc(c);
#pragma unroll
                for (int tp = 0; tp < TPL; ++tp) {
                    const int t = l + 64 * tp;
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
                        x.vr[tp][hf] = buf_raw_frag<TIn>(
                            r_v, (int)((uint32_t)(t * row_v) + (uint32_t)(8 * hf * ES) + pad_if(t < CP)));
                    x.sa[tp] = buf_elem<float>(rs, (int)((uint32_t)(4 * t) + pad_if(t < CP)));
                    x.ss[tp] = buf_elem<float>(rs, (int)((uint32_t)(4 * (CP + t)) + pad_if(t < CP)));
                }
                x.gc = buf_elem<float>(rs, 3 * CP * 4);
            }
        };
        auto store_stage = [&](const OS& x, int par) {
            if constexpr (SG::TLDS) {
#pragma unroll
                for (int m = 0; m < NTS; ++m) {
                    const int pi = ow + NOW * m;
                    if (pi < 2 * NTRI) s_tf[par][pi][l] = x.tst[m];
                }
            }
            if (stager) {
#pragma unroll
                for (int tp = 0; tp < TPL; ++tp) {
                    const int t = l + 64 * tp;  // < CPV; slots past CP hold zeros
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                        for (int e = 0; e < 8; ++e) s_vt[par][8 * hf + e][t] = elem_f32(x.vr[tp][hf], e);
                    s_sc[par][0][t] = x.sa[tp];
                    s_sc[par][1][t] = x.ss[tp];
                }
                s_gc[par] = x.gc;  // every lane writes the same value
            }
        };
        auto load = [&](OS& x, int64_t j) {
            {
                const auto r = qk_rsrc(q, clampc(j));
#pragma unroll
                for (int i = 0; i < RTO; ++i)
#pragma unroll
                    for (int kt = 0; kt < KTD; ++kt) x.qr[i][kt] = buf_raw_frag<TIn>(r, qk_off(ow + NOW * i, kt));
            }
            {
                const int64_t c = clampc(j - 1);
                const auto r = make_rsrc(ws + L.pt + vh_of(c) * G::TRI_BYTES, G::TRI_BYTES);
                const auto rs = sc_rsrc(c);
#pragma unroll
                for (int i = 0; i < RTO; ++i) {
                    const int rt = ow + NOW * i;
#pragma unroll
                    for (int kt = 0; kt < KTC; ++kt) {
                        const bool ok = rt < RT && 2 * kt <= rt;
                        const int o = (tri_off(rt) + kt) * 2048 + l * 16;
                        x.pf[i][kt][0] = buf_bf16x8(r, ok ? o : (int)OOR);
                        x.pf[i][kt][1] = buf_bf16x8(r, ok ? o + 1024 : (int)OOR);
                    }
                    x.ov[i] = buf_elem<float>(rs, rt < RT ? 2 * CP * 4 + (16 * rt + lr) * 4 : (int)OOR);
                }
            }
            load_stage(x, j + 1);
        };
        // Outputs are formed transposed, O^T = (Q M0)^T diag(o) + U^T Ptil^T, as 16 value
        // channels x 16 tokens tiles: the state and U fragments serve unchanged as A
        // operands and the Q row fragments as B operands, Ptil^T arrives as B fragments, and
        // each lane ends up with four consecutive channels of one token (one 16-byte store).
        auto do_out = [&](const OS& x, int64_t c) {
            const int par = (int)(c & 1);
            floatx4 urow[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) urow[rt] = s_uf[par][rt][l];
            bf16x8 ufr[KTC][2];
            rows_to_frags<RT, KTC>(urow, ufr);
            const auto r_o = make_rsrc(out + (tok0_of(c) * h_v + h) * (int64_t)D + cb * 16,
                                       (rows_of(c) - 1) * row_o + 64);
#pragma unroll
            for (int i = 0; i < RTO; ++i) {
                const int rt = ow + NOW * i;
                if (rt >= RT) continue;
                floatx4 acc = x.ov[i] * qm[i];
#pragma unroll
                for (int kt = 0; kt < KTC; ++kt)
                    if (2 * kt <= rt) acc = mfma_split<2, 2>(ufr[kt], x.pf[i][kt], acc);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), r_o,
                                                       (int)((16 * rt + lr) * row_o) + lg * 16, 0, 0);
            }
        };
        // (Q M0)^T of chunk c, the state from LDS.
        auto do_qm = [&](const OS& x, int64_t c) {
            const int par = (int)(c & 1);
            bf16x8 mfr[KTD][2];
#pragma unroll
            for (int kt = 0; kt < KTD; ++kt)
#pragma unroll
                for (int p = 0; p < 2; ++p) mfr[kt][p] = s_mf[par][kt][p][l];
#pragma unroll
            for (int i = 0; i < RTO; ++i) {
                if (ow + NOW * i >= RT) continue;
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; kt < KTD; ++kt) {
                    bf16x8 qa[NS];
                    to_pieces(x.qr[i][kt], qa);
                    acc = mfma_split<2, NS>(mfr[kt], qa, acc);
                }
                qm[i] = acc;
            }
        };
        auto window = [&](const OS& x, int64_t j) {
            store_stage(x, (int)((j + 1) & 1));  // for the chain waves' chunk j + 1
            if (j >= 1) do_out(x, j - 1);
            if (j < nch) do_qm(x, j);
        };

        {
            OS s0;
            load_stage(s0, 0);
            settle();
            store_stage(s0, 0);
        }
        OS A;
        load(A, 0);
        if constexpr (SG::DB) {
            OS B;
            settle();
            for (int64_t j = 0;;) {
                load(B, j + 1);
                __syncthreads();
                window(A, j);
                settle();
                if (++j > nch) break;
                load(A, j + 1);
                __syncthreads();
                window(B, j);
                settle();
                if (++j > nch) break;
            }
        } else {
#pragma unroll 1
            for (int64_t j = 0; j <= nch; ++j) {
                if (j > 0) load(A, j);
                __syncthreads();
                window(A, j);
                settle();
            }
        }
    }
}

// ================================================== scan, 64-token chunks, bf16, d_k = d_v = 128
// The sequential pass for the workload this library is tuned for (bf16 q/k/v, 128-wide
// heads, 64-token chunks). One workgroup of eight waves per (sequence, V head, 16 value
// channels); wave w runs on SIMD w mod 4:
//   chain waves 0, 1 (SIMDs 0, 1): each holds one d_k half of the state (64 features x 16
//        channels) in MFMA accumulators and runs the whole recurrence of every chunk from
//        operands in LDS or registers, with one exchange of partial products per chunk:
//          P_c = K_c M_c (the halves' parts summed in a fixed order, so both waves form the
//          same X and U), X = V - diag(a) P_c, U = T' X, W = diag(s) U,
//          M_{c+1} = Gamma_C M_c + K_c^T W, then its part of P_{c+1} = K_{c+1} M_{c+1} and
//          the K_{c+1}^T fragments of the next update, read from LDS while K_{c+1} is there;
//   output waves 2, 3 (SIMDs 2, 3): one window behind, O^T = (Q M_c)^T diag(o) + U^T Ptil^T
//        for two 16-token row tiles each (tiles 0 and 3, 1 and 2: equal triangular work),
//        with the Ptil pieces loaded straight into registers a window ahead;
//   staging waves 4..7 (one per SIMD): every other input straight into LDS one window ahead
//        of use (loads that write LDS directly), into rings of two chunks.
// Every ring and exchange slot is indexed by chunk parity, and the loops take two windows
// per iteration, so every LDS address is fixed at compile time. The chain waves also touch,
// every window, one cache line per lane of the inputs of the chunk eight ahead (shared out
// over the workgroups that read them), so that the staging loads hit L2.
// Windows are separated by workgroup barriers, one per chunk: window -1 forms the state's
// first partial products; windows 0 .. nwin - 1 the chunks, where nwin is the chunk count
// rounded up to even (the extra window, when there is one, has a = s = 0 and Gamma_C = 1
// staged, so that it leaves the state unchanged: M <- 1 * M + K^T 0); a last window the last
// outputs.
// Staged data of chunks past the sequence is the last chunk's again (or zero scalars), in
// slots whose products nobody reads. The rings start cleared, so rows past a short last
// chunk (never written: their loads fall outside the buffer range) hold finite values, which
// meet zero coefficients (a, s, T', Ptil are zero for tokens past the sequence).
namespace c64 {
constexpr int D = 128, C = 64;
constexpr int RT = 4;        // 16-token row tiles of a chunk
constexpr int KTC = 2;       // token k tiles (32) of a chunk
constexpr int KTH = 2;       // feature k tiles (32) per chain wave
constexpr int MTH = 4;       // 16-feature state tiles per chain wave
constexpr int NTRI = 6;      // stored lower-triangular 16 x 32 tiles of T' and Ptil
constexpr int ROWB = 256;    // bytes per staged bf16 row of 128 features
constexpr int K_BYTES = C * ROWB;  // one chunk of staged K (or Q) rows
constexpr int NSTG = 4;      // staging waves
constexpr int NKI = C * ROWB / 1024;  // 1 KB row loads per chunk (4 rows each)
constexpr int TOUCH_AHEAD = 8;
}  // namespace c64

template <int P>
using parity_t = std::integral_constant<int, P>;

__global__ void __launch_bounds__(512)
chunk64_scan_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, const char* __restrict__ ws, ChunkWs L,
                    const float* state_in, float* __restrict__ out, float* state_out, int64_t T,
                    int h_qk, int h_v, int64_t nblocks)
{
    using namespace c64;
    using G = Geo<D, C, false>;
    static_assert(G::NTRI == NTRI && G::RT == RT && G::KTC == KTC && G::KTH == KTH &&
                  G::MTH == MTH && G::H_BYTES == 0, "geometry of the prepared workspace");
    constexpr int ES = 2;
    constexpr int RPB = 256 / ROWB;  // staged rows per 64 LDS banks (1)
    constexpr int NG = ROWB / 16;    // 16-byte granules per staged row
    constexpr int RPI = 4;           // staged rows per 1 KB load

    // LDS, every ring and exchange by chunk parity
    __shared__ __align__(16) char s_k[2][K_BYTES];             // K rows (swizzled granules)
    __shared__ __align__(16) char s_q[2][K_BYTES];             // Q rows (swizzled granules)
    __shared__ __align__(16) bf16x8 s_tf[2][2 * NTRI][64];     // T' pieces (hi, lo)
    __shared__ __align__(16) char s_v[2][C * 32];              // V block: 64 tokens x 16 bf16
    __shared__ __align__(16) float s_sc[2][256];               // a, s, o, Gamma_C
    __shared__ __align__(16) floatx4 s_pp[2][2][RT][64];       // each chain wave's part of K M
    __shared__ __align__(16) bf16x8 s_mf[2][2 * KTH][2][64];   // the state as B fragments
    __shared__ __align__(16) floatx4 s_uf[2][RT][64];          // U (accumulator layout)

    int64_t lin = blockIdx.x;
    if (nblocks % 8 == 0) lin = (int64_t)(blockIdx.x % 8) * (nblocks / 8) + blockIdx.x / 8;
    const int cb = (int)(lin % (D / 16));
    const int64_t nh = lin / (D / 16);
    const int64_t seq = nh / h_v;
    const int h = (int)(nh - seq * h_v);
    const int hq = h / (h_v / h_qk);
    const int tid = threadIdx.x, l = tid & 63, lr = l & 15, lg = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t nch = L.nch;
    const int64_t nwin = nch + (nch & 1);

    const int64_t row_qk = (int64_t)h_qk * D * ES;
    const int64_t row_v = (int64_t)h_v * D * ES;
    const int64_t row_o = (int64_t)h_v * D * 4;
    auto clampc = [&](int64_t c) { return c < 0 ? 0 : (c < nch ? c : nch - 1); };
    auto tok0_of = [&](int64_t c) { return seq * T + c * C; };
    auto rows_of = [&](int64_t c) { return (T - c * C) < C ? (T - c * C) : (int64_t)C; };
    auto vh_of = [&](int64_t c) { return (size_t)((seq * nch + c) * h_v + h); };
    auto srow = [&](int r, int j) { return r * ROWB + 16 * (j ^ swz<RPB>(r)); };

    // Clear the staged rows and V blocks once (see above). 512 threads, 16 bytes each.
    for (int o = 16 * tid; o < 2 * K_BYTES; o += 16 * 512) {
        *reinterpret_cast<u32x4*>(&s_k[0][0] + o) = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(&s_q[0][0] + o) = u32x4{0u, 0u, 0u, 0u};
    }
    for (int o = 16 * tid; o < 2 * C * 32; o += 16 * 512)
        *reinterpret_cast<u32x4*>(&s_v[0][0] + o) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();

    if (w < 2) {
        // ======================================================= chain wave hh
        const int hh = w;
        const int64_t sbase = nh * (int64_t)D * D;
        auto st_off = [&](int mt, int e) {
            const int f = feat_of(mt, 4 * lg + e);
            return (int)((f * D + cb * 16 + lr) * 4);
        };
        floatx4 macc[MTH];  // state tiles MTH hh + i
        {
            const auto r = make_rsrc(state_in + (state_in ? sbase : 0), state_in ? (int64_t)D * D * 4 : 0);
#pragma unroll
            for (int i = 0; i < MTH; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) macc[i][e] = buf_elem<float>(r, st_off(MTH * hh + i, e));
        }
        bf16x8 mf[KTH][2];
        auto split_state = [&]() {
#pragma unroll
            for (int kk = 0; kk < KTH; ++kk) pair_to_frag(macc[2 * kk], macc[2 * kk + 1], mf[kk][0], mf[kk][1]);
        };
        bf16x8 kts[MTH][KTC];  // K^T A fragments of the chunk the next update uses
        bf16x8 ka[RT][KTH];    // K row A fragments (this wave's features) of the next chunk
        // From K ring slot S (the chunk after the current one): its K rows and K^T fragments
        // (two transposing reads each, token slots 0..3 and 4..7) into registers.
        auto read_next_k = [&](auto slot_c, bf16x8 (*ktn)[KTC]) {
            constexpr int S = decltype(slot_c)::value;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kk = 0; kk < KTH; ++kk)
                    ka[rt][kk] = *reinterpret_cast<const bf16x8*>(s_k[S] + srow(16 * rt + lr, 4 * (KTH * hh + kk) + lg));
#pragma unroll
            for (int i = 0; i < MTH; ++i)
#pragma unroll
                for (int kt = 0; kt < KTC; ++kt) {
                    const int r = 32 * kt + 4 * lg + (lr >> 2);
                    const int j = 4 * (KTH * hh + (i >> 1)) + (lr & 3);
                    const char* base = s_k[S] + 8 * (i & 1);
                    const bf16x4 x0 = lds_read_tr16(base + srow(r, j));
                    const bf16x4 x1 = lds_read_tr16(base + srow(r + 16, j));
                    ktn[i][kt] = bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
                }
        };
        floatx4 pp[RT];  // this wave's part of K M for the chunk about to be processed
        // This wave's part of K M for the next chunk (K rows in ka), published with the state
        // fragments in exchange slot S.
        auto publish_next = [&](auto slot_c) {
            constexpr int S = decltype(slot_c)::value;
#pragma unroll
            for (int kk = 0; kk < KTH; ++kk)
#pragma unroll
                for (int p = 0; p < 2; ++p) s_mf[S][KTH * hh + kk][p][l] = mf[kk][p];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KTH; ++kk) acc = mfma_split<1, 2>(&ka[rt][kk], mf[kk], acc);
                pp[rt] = acc;
                s_pp[S][hh][rt][l] = acc;
            }
        };

        // Cache-line touches: one 128-byte line per lane of a chunk's inputs. K and Q rows go
        // round the workgroups of the QK head, workspace blocks and V rows round the
        // workgroups of the V head; lanes past this workgroup's share touch lane 0's line.
        // The lane's line in chunk j is touch_base + j * touch_step (full chunks; a partial
        // last chunk is touched as the chunk before it).
        uint64_t touch_base, touch_step;
        {
            constexpr int LPR128 = (D * ES + 127) / 128;
            constexpr int NCB = D / 16;
            constexpr int TL = (int)(G::TRI_BYTES / 128);
            constexpr int SCL = (int)((G::SC_BYTES + 127) / 128) - 1;
            constexpr int NWS = 2 * TL + SCL;
            constexpr int HALF = C * LPR128;
            auto pick = [](bool cond, uint64_t x, uint64_t y) {
                const uint64_t m = 0 - (uint64_t)cond;
                return (x & m) | (y & ~m);
            };
            const int grp = h_v / h_qk, nbq = grp * NCB, iq = (h % grp) * NCB + cb;
            const int nq_mine = (2 * HALF - iq + nbq - 1) / nbq;
            const int nv_mine = (NWS + HALF - cb + NCB - 1) / NCB;
            // the second chain wave touches lane 0's line only (its loop issues the same
            // loads as the first's, see below, but need not repeat its requests). The lines
            // of T', Ptil and the scalars are touched only when the call's workspace exceeds
            // 64 MiB: a smaller one, which the preparation has just written, is still in the
            // 256 MB MALL, and touching it only costs vector-memory issue (measured: 4K
            // tokens, 51 MB of workspace, 1.8 us faster per layer without those touches; 8K,
            // 102 MB, equal; 16K, 204 MB, 11% slower without).
            const bool touch_ws = L.total > ((size_t)64 << 20);
            const bool wsline = l >= nq_mine && cb + NCB * (l - nq_mine) < NWS;
            const int li = (l < nq_mine + nv_mine && hh == 0 && (touch_ws || !wsline)) ? l : 0;
            const bool isq = li < nq_mine;
            const int lq = iq + nbq * li, rq = lq < HALF ? lq : lq - HALF;
            const uint64_t q0 = pick(lq < HALF, (uint64_t)k, (uint64_t)q) +
                                (uint64_t)(((seq * T + rq / LPR128) * h_qk + hq) * (int64_t)D * ES + 128 * (rq % LPR128));
            const uint64_t qs = (uint64_t)C * h_qk * D * ES;
            const int lv = isq ? 0 : cb + NCB * (li - nq_mine);
            const uint64_t vh0 = (uint64_t)(seq * nch * h_v + h), wsb = (uint64_t)ws;
            const uint64_t w_tt = wsb + L.tt + vh0 * G::TRI_BYTES + 128 * lv;
            const uint64_t w_pt = wsb + L.pt + vh0 * G::TRI_BYTES + 128 * (lv - TL);
            const uint64_t w_sc = wsb + L.sc + vh0 * G::SC_BYTES + 128 * (lv - 2 * TL);
            uint64_t w0 = pick(lv < 2 * TL, w_pt, w_sc);
            uint64_t ws_step = pick(lv < 2 * TL, (uint64_t)h_v * G::TRI_BYTES, (uint64_t)h_v * G::SC_BYTES);
            w0 = pick(lv < TL, w_tt, w0);
            const int rv = lv - NWS;
            const uint64_t v0 = (uint64_t)v + (uint64_t)(((seq * T + rv / LPR128) * h_v + h) * (int64_t)D * ES + 128 * (rv % LPR128));
            const uint64_t vs = (uint64_t)C * h_v * D * ES;
            touch_base = pick(isq, q0, pick(lv < NWS, w0, v0));
            touch_step = pick(isq, qs, pick(lv < NWS, ws_step, vs));
        }
        // the last chunk touched: the last full one (the sequence's only, partial, chunk: none)
        const int64_t tlast = rows_of(nch - 1) == C ? nch - 1 : nch - 2;
        const uint64_t touch_first = tlast >= 0 ? touch_base : (uint64_t)ws;
        uint64_t touch_at = touch_first + (uint64_t)(tlast < TOUCH_AHEAD ? (tlast > 0 ? tlast : 0) : TOUCH_AHEAD) * touch_step;

        split_state();
        barrier_lds_only();               // K rows of chunk 0 staged
        read_next_k(parity_t<0>{}, kts);  // window -1: K_0 and K_0^T
        publish_next(parity_t<0>{});      // this wave's part of K_0 M_0

        // One chunk. Every LDS read of the window is issued right after its barrier: the
        // partner's partial products, V and a (which X waits for) first, then T', s and the
        // next chunk's K rows and K^T fragments (its ring slot is stable all window), so that
        // one LDS round trip precedes X and the last products wait for no read. The work
        // then runs by token k tile, so that the hi/lo splits of one tile overlap the
        // products of the other.
        auto window = [&](auto par_c, int64_t c, uint32_t& touched) {
            constexpr int PAR = decltype(par_c)::value;  // c & 1
            barrier_lds_only();
            floatx4 po[RT], vv[RT], av[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                po[rt] = s_pp[PAR][hh ^ 1][rt][l];
                const bf16x4 vr = lds_read_tr16(s_v[PAR] + (16 * rt + 4 * lg + (lr >> 2)) * 32 + 8 * (lr & 3));
                vv[rt] = floatx4{(float)vr[0], (float)vr[1], (float)vr[2], (float)vr[3]};
                av[rt] = *reinterpret_cast<const floatx4*>(&s_sc[PAR][16 * rt + 4 * lg]);
            }
            bf16x8 tf[2 * NTRI];
#pragma unroll
            for (int pi = 0; pi < 2 * NTRI; ++pi) tf[pi] = s_tf[PAR][pi][l];
            floatx4 sv[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) sv[rt] = *reinterpret_cast<const floatx4*>(&s_sc[PAR][C + 16 * rt + 4 * lg]);
            const float gc = s_sc[PAR][3 * C];
            bf16x8 ktn[MTH][KTC];
            read_next_k(parity_t<PAR ^ 1>{}, ktn);  // chunk c + 1 (past the last: never used)
            // X = V - diag(a) K M, the two parts added in the order chain 0 + chain 1, as B
            // fragments by token k tile
            bf16x8 xf[KTC][2];
#pragma unroll
            for (int kt = 0; kt < KTC; ++kt) {
                floatx4 x2[2];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int rt = 2 * kt + hf;
                    const floatx4 z = hh == 0 ? pp[rt] + po[rt] : po[rt] + pp[rt];
                    x2[hf] = vv[rt] - av[rt] * z;
                }
                pair_to_frag(x2[0], x2[1], xf[kt][0], xf[kt][1]);
            }
            // U = T' X (lower triangular: row tile rt uses token k tiles 0 .. rt / 2),
            // W = diag(s) U, then M <- Gamma_C M + K^T W, token k tile by token k tile
            floatx4 u[RT];
            bf16x8 wf[KTC][2];
            auto u_tile = [&](int rt) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; 2 * kt <= rt; ++kt) acc = mfma_split<2, 2>(&tf[2 * (tri_off(rt) + kt)], xf[kt], acc);
                u[rt] = acc;
            };
            auto w_frag = [&](int kt) {
                const floatx4 w0 = u[2 * kt] * sv[2 * kt], w1 = u[2 * kt + 1] * sv[2 * kt + 1];
                pair_to_frag(w0, w1, wf[kt][0], wf[kt][1]);
            };
            u_tile(0);
            u_tile(1);
            w_frag(0);
            u_tile(2);
            u_tile(3);
#pragma unroll
            for (int i = 0; i < MTH; ++i) macc[i] = mfma_split<1, 2>(&kts[i][0], wf[0], gc * macc[i]);
            w_frag(1);
            if (hh == 0) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) s_uf[PAR][rt][l] = u[rt];
            }
#pragma unroll
            for (int i = 0; i < MTH; ++i) macc[i] = mfma_split<1, 2>(&kts[i][1], wf[1], macc[i]);
            split_state();
            publish_next(parity_t<PAR ^ 1>{});  // chunk c + 1 (past the last: never read)
#pragma unroll
            for (int i = 0; i < MTH; ++i)
#pragma unroll
                for (int kt = 0; kt < KTC; ++kt) kts[i][kt] = ktn[i][kt];
            // Touch the lines of chunk c + 8 after the touch of window c - 2 has landed. Both
            // chain waves issue a touch (with no branch around it, the wait for the earlier
            // touch is exact: this wave issues no other vector memory operations in the loop).
            asm volatile("" ::"v"(touched));
            touched = *(const __attribute__((address_space(1))) uint32_t*)touch_at;
            if (c + TOUCH_AHEAD < tlast) touch_at += touch_step;  // wave-uniform
        };
        uint32_t ta = 0, tb = 0;
#pragma unroll 1
        for (int64_t c = 0; c < nwin; c += 2) {
            window(parity_t<0>{}, c, ta);
            window(parity_t<1>{}, c + 1, tb);
        }
        barrier_lds_only();  // the last window
        asm volatile("" ::"v"(ta), "v"(tb));
        {
            const auto r = make_rsrc(state_out + sbase, (int64_t)D * D * 4);
#pragma unroll
            for (int i = 0; i < MTH; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(macc[i][e]), r, st_off(MTH * hh + i, e), 0, 0);
        }
    } else if (w < 4) {
        // ======================================================= output wave
        // Row tiles OW and 3 - OW (equal triangular work), fixed at compile time.
        auto output_wave = [&](auto owc) {
            constexpr int OW = decltype(owc)::value;
            constexpr int RTS[2] = {OW, 3 - OW};
            floatx4 qm[2];         // (Q M_c)^T of the chunk being finished
            float ov[2];           // o of token lr of each row tile of that chunk
            bf16x8 pf[2][KTC][2];  // its Ptil^T pieces: [row tile][token k tile][hi, lo]
            auto start_chunk = [&](auto par_c, int64_t c) {
                constexpr int PAR = decltype(par_c)::value;
                const auto r = make_rsrc(ws + L.pt + vh_of(c) * G::TRI_BYTES, G::TRI_BYTES);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int kt = 0; kt < KTC; ++kt) {
                        if (2 * kt > RTS[i]) continue;
                        const int o = (tri_off(RTS[i]) + kt) * 2048 + l * 16;
                        pf[i][kt][0] = buf_bf16x8(r, o);
                        pf[i][kt][1] = buf_bf16x8(r, o + 1024);
                    }
                bf16x8 mfr[2 * KTH][2];
#pragma unroll
                for (int kt = 0; kt < 2 * KTH; ++kt)
#pragma unroll
                    for (int p = 0; p < 2; ++p) mfr[kt][p] = s_mf[PAR][kt][p][l];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    ov[i] = s_sc[PAR][2 * C + 16 * RTS[i] + lr];
                    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kt = 0; kt < 2 * KTH; ++kt) {
                        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(s_q[PAR] + srow(16 * RTS[i] + lr, 4 * kt + lg));
                        acc = mfma_split<2, 1>(mfr[kt], &qa, acc);
                    }
                    qm[i] = acc;
                }
            };
            // O^T = U^T Ptil^T + (Q M)^T diag(o), 16 value channels x 16 tokens per row tile:
            // each lane ends up with four consecutive channels of one token (one 16-byte store).
            auto finish_chunk = [&](auto par_c, int64_t c) {
                constexpr int PAR = decltype(par_c)::value;
                floatx4 urow[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) urow[rt] = s_uf[PAR][rt][l];
                bf16x8 ufr[KTC][2];
                rows_to_frags<RT, KTC>(urow, ufr);
                const auto r_o = make_rsrc(out + (tok0_of(c) * h_v + h) * (int64_t)D + cb * 16,
                                           (rows_of(c) - 1) * row_o + 64);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    floatx4 acc = ov[i] * qm[i];
#pragma unroll
                    for (int kt = 0; kt < KTC; ++kt)
                        if (2 * kt <= RTS[i]) acc = mfma_split<2, 2>(ufr[kt], pf[i][kt], acc);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), r_o,
                                                           (int)((16 * RTS[i] + lr) * row_o) + lg * 16, 0, 0);
                }
            };
            // window c: finish chunk c - 1, start chunk c
            auto window = [&](auto par_c, int64_t c) {
                constexpr int PAR = decltype(par_c)::value;
                barrier_lds_only();
                if (c >= 1 && c <= nch) finish_chunk(parity_t<PAR ^ 1>{}, c - 1);
                if (c < nch) start_chunk(par_c, c);
            };
            barrier_lds_only();  // window -1
#pragma unroll 1
            for (int64_t c = 0; c < nwin; c += 2) {
                window(parity_t<0>{}, c);
                window(parity_t<1>{}, c + 1);
            }
            window(parity_t<0>{}, nwin);  // the last window
            __builtin_amdgcn_s_waitcnt(0);
        };
        if (w == 2) output_wave(std::integral_constant<int, 0>{});
        else output_wave(std::integral_constant<int, 1>{});
    } else {
        // ======================================================= staging wave hs
        const int hs = w - 4;
        auto qk_rsrc = [&](const uint16_t* base, int64_t c) {
            return make_rsrc(base + (tok0_of(c) * h_qk + hq) * (int64_t)D, (rows_of(c) - 1) * row_qk + D * ES);
        };
        // K or Q rows of chunk c straight into `dst`: load m covers staged rows 4 mi .. 4 mi + 3
        // (mi = hs + NSTG m), 1 KB, lane l landing at byte 16 l of it.
        auto dma_rows = [&](const uint16_t* base, int64_t c, char* dst) {
            const auto r = qk_rsrc(base, clampc(c));
#pragma unroll
            for (int m = 0; m < NKI / NSTG; ++m) {
                const int mi = hs + NSTG * m;
                const int row = RPI * mi + l / NG, pos = l % NG;
                const int g = pos ^ swz<RPB>(row);
                load_to_lds(r, dst + mi * 1024, (int)((uint32_t)(row * row_qk) + (uint32_t)(16 * g)));
            }
        };
        // window c stages what window c + 1 reads: K rows of chunk c + 2 (into the slot of
        // chunk c, whose reads ended in window c - 1), and the Q rows, T' pieces, V block
        // and scalars of chunk c + 1. Chunks past the sequence: the last chunk's rows and
        // pieces again, and scalars a = s = 0, Gamma_C = 1 (an update that changes nothing;
        // every scalar the chain reads is written, since 0 times a stale non-finite value
        // would not be zero).
        auto stage = [&](auto par_c, int64_t c) {
            constexpr int PAR = decltype(par_c)::value;  // c & 1
            constexpr int NXT = PAR ^ 1;                 // (c + 1) & 1
            const int64_t j = c + 1, jc = clampc(j);
            dma_rows(k, c + 2, s_k[PAR]);
            dma_rows(q, j, s_q[NXT]);
            {
                const auto r = make_rsrc(ws + L.tt + vh_of(jc) * G::TRI_BYTES, G::TRI_BYTES);
#pragma unroll
                for (int m = 0; hs + NSTG * m < 2 * NTRI; ++m)
                    load_to_lds(r, s_tf[NXT][hs + NSTG * m], (hs + NSTG * m) * 1024 + l * 16);
            }
            if (hs == 0) {
                const auto r_v = make_rsrc(v + (tok0_of(jc) * h_v + h) * (int64_t)D + cb * 16,
                                           (rows_of(jc) - 1) * row_v + 32);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int t = 32 * m + l / 2;
                    load_to_lds(r_v, s_v[NXT] + m * 1024, (int)((uint32_t)(t * row_v) + (uint32_t)(16 * (l & 1))));
                }
            } else if (hs == 1) {
                if (j < nch) {
                    load_to_lds(make_rsrc(ws + L.sc + vh_of(j) * G::SC_BYTES, G::SC_BYTES), s_sc[NXT], 16 * l);
                } else {
                    s_sc[NXT][l] = 0.f;
                    s_sc[NXT][C + l] = 0.f;
                    if (l == 0) s_sc[NXT][3 * C] = 1.f;
                }
            }
        };
        dma_rows(k, 0, s_k[0]);
        __builtin_amdgcn_s_waitcnt(0);
        barrier_lds_only();  // window -1
        stage(parity_t<1>{}, -1);
        __builtin_amdgcn_s_waitcnt(0);  // this window's loads have landed in LDS
#pragma unroll 1
        for (int64_t c = 0; c < nwin; c += 2) {
            barrier_lds_only();
            stage(parity_t<0>{}, c);
            __builtin_amdgcn_s_waitcnt(0);
            barrier_lds_only();
            stage(parity_t<1>{}, c + 1);
            __builtin_amdgcn_s_waitcnt(0);
        }
        barrier_lds_only();  // the last window
    }
}

// Compute units of the current device, looked up once per device (0 if the query fails).
int device_cu_count()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 0;
    }
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            return 0;
        }
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int D, int C, typename TIn>
hipError_t launch_chunked_t(const Call& cl, int parts)
{
    constexpr bool F32IN = std::is_same<TIn, float>::value;
    const ChunkWs L = chunk_ws(cl.n, cl.t, cl.h_qk, cl.h_v, D, C, F32IN);
    char* ws = static_cast<char*>(cl.ws);
    const TIn* q = static_cast<const TIn*>(cl.q);
    const TIn* k = static_cast<const TIn*>(cl.k);
    const TIn* v = static_cast<const TIn*>(cl.v);
    const int64_t prep_blocks = cl.n * L.nch * cl.h_qk;
    if (parts & kChunkPrep) {
        // The staggered start of chunk_prep_kernel, measured for 64-token chunks of bf16 rows
        // of 128 features (four workgroups resident per CU): 1,024 workgroups at 4K tokens,
        // 25.0 -> 24.0 us with about 1.5-2 us per group (0.5 us per group: no change; 3 us:
        // slower). Only when the whole grid is resident at once and spans several groups.
        int stagger_wgs = 1, stagger_units = 0;
        bool per_head = false;
        if constexpr (C == 64 && D == 128 && !F32IN) {
            const int cus = device_cu_count();
            // A workgroup per V head (all four waves on it) where that duplicates nothing (one
            // V head per QK head) or where the grid would leave CUs idle, so that one
            // workgroup's latency rather than the chip's throughput sets the time.
            per_head = cus > 0 && (cl.h_v == cl.h_qk || prep_blocks <= cus);
            // (the stagger, measured for four resident workgroups per CU, only on that grid)
            const bool same_grid = !per_head || cl.h_v == cl.h_qk;
            if (same_grid && cus > 0 && prep_blocks > cus && prep_blocks <= 4 * (int64_t)cus) {
                stagger_wgs = cus;
                // one group's q/k rows (cus x 2 x C x D x 2 bytes) at about 5 TB/s, in
                // s_sleep units of 64 clocks at about 2.1 GHz
                stagger_units = (int)((double)cus * 2 * C * D * sizeof(TIn) / 5.0e12 * 2.1e9 / 64.0);
            }
        }
        if constexpr (C == 64 && D == 128 && !F32IN) {
            if (per_head) {
                hipLaunchKernelGGL((chunk_prep_kernel<D, C, TIn, true>), dim3((unsigned)(cl.n * L.nch * cl.h_v)),
                                   dim3(256), 0, cl.stream, q, k, cl.g, cl.beta, ws, L, cl.t, cl.h_qk,
                                   cl.h_v, cl.eps, stagger_wgs, stagger_units);
            }
        }
        if (!per_head) {
            hipLaunchKernelGGL((chunk_prep_kernel<D, C, TIn>), dim3((unsigned)prep_blocks), dim3(256), 0,
                               cl.stream, q, k, cl.g, cl.beta, ws, L, cl.t, cl.h_qk, cl.h_v, cl.eps,
                               stagger_wgs, stagger_units);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (!(parts & kChunkScan)) return hipSuccess;
    const int64_t scan_blocks = cl.n * cl.h_v * (D / 16);
    if constexpr (C <= 32) {
        hipLaunchKernelGGL((chunk_scan_kernel<D, C, TIn>), dim3((unsigned)scan_blocks),
                           dim3(ScanGeo<D, C, TIn>::THREADS), 0, cl.stream, q, k, v, ws, L,
                           cl.state_in, cl.out, cl.state_out, cl.t, cl.h_qk, cl.h_v, scan_blocks);
    } else if constexpr (C == 64 && D == 128 && !F32IN) {
        hipLaunchKernelGGL(chunk64_scan_kernel, dim3((unsigned)scan_blocks), dim3(512), 0, cl.stream,
                           q, k, v, ws, L, cl.state_in, cl.out, cl.state_out, cl.t, cl.h_qk,
                           cl.h_v, scan_blocks);
    } else {
        hipLaunchKernelGGL((chunk_scan_wide_kernel<D, C, TIn>), dim3((unsigned)scan_blocks), dim3(256), 0,
                           cl.stream, q, k, v, ws, L, cl.state_in, cl.out, cl.state_out, cl.t,
                           cl.h_qk, cl.h_v, scan_blocks);
    }
    return hipGetLastError();
}

template <int D, typename TIn>
hipError_t dispatch_c(const Call& cl, int chunk, int parts)
{
    switch (chunk) {
        case 16: return launch_chunked_t<D, 16, TIn>(cl, parts);
        case 32: return launch_chunked_t<D, 32, TIn>(cl, parts);
        case 64: return launch_chunked_t<D, 64, TIn>(cl, parts);
        case 128: return launch_chunked_t<D, 128, TIn>(cl, parts);
        default: return hipErrorInvalidValue;
    }
}

template <typename TIn>
hipError_t dispatch_d(const Call& cl, int chunk, int parts)
{
    switch (cl.d) {
        case 16: return dispatch_c<16, TIn>(cl, chunk, parts);
        case 32: return dispatch_c<32, TIn>(cl, chunk, parts);
        case 64: return dispatch_c<64, TIn>(cl, chunk, parts);
        case 128: return dispatch_c<128, TIn>(cl, chunk, parts);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t chunked_workspace_bytes(int64_t n, int64_t t, int32_t h_qk, int32_t h_v, int32_t d,
                               int chunk, int32_t dtype)
{
    return chunk_ws(n, t, h_qk, h_v, d, chunk, dtype != GDN_BF16).total;
}

hipError_t launch_chunked(const Call& c, int chunk, int parts)
{
    return c.dtype == GDN_BF16 ? dispatch_d<uint16_t>(c, chunk, parts)
                               : dispatch_d<float>(c, chunk, parts);
}

}  // namespace gdn
