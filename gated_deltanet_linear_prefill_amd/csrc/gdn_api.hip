// gdn_api.hip -- the C ABI of libgdn.so (declared and documented in include/gdn.h):
// host-side validation, workspace sizing, method choice and kernel dispatch.
//
// Every check runs on the host before the first HIP call, so each error path is testable
// without a GPU, and on error nothing is enqueued.
#include <mutex>
#include <vector>
#include <math.h>
#include <string.h>

#include "gdn_internal.hpp"

// A recorded decode graph: the instantiated HIP graph it replays.
struct gdn_graph_rec {
    hipGraphExec_t exec;
};

namespace gdn {
namespace {

#include "gdn_crossover.inc"  // kCrossover[]: measured scan/chunk choice by length

struct Range {
    uintptr_t lo, hi;  // [lo, hi); empty when lo == hi
};

bool overlap(Range a, Range b)
{
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool mul_ok(int64_t a, int64_t b, int64_t* r)
{
    return !__builtin_mul_overflow(a, b, r);
}

bool supported_d(int32_t d)
{
    return d == 16 || d == 32 || d == 64 || d == 128;
}

bool supported_chunk(int32_t c)
{
    return c == 16 || c == 32 || c == 64 || c == 128;
}

// Element counts of every tensor, or false on overflow. Sizes are bounded so that every
// byte offset fits in int64 and every grid dimension in 31 bits.
struct Sizes {
    int64_t qk, v, gb, state, out;  // elements
    size_t esize;                   // bytes per q/k/v element
};

gdn_status check_dims(const gdn_dims* d, Sizes* s)
{
    if (!d) return GDN_ERR_NULL;
    if (d->n < 0 || d->t < 0 || d->h_qk <= 0 || d->h_v <= 0 || d->d_k <= 0 || d->d_v <= 0)
        return GDN_ERR_SHAPE;
    if (d->h_v % d->h_qk != 0) return GDN_ERR_SHAPE;
    if (!(d->l2_eps >= 0.0f) || !isfinite(d->l2_eps)) return GDN_ERR_SHAPE;
    if (d->qkv_dtype != GDN_F32 && d->qkv_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (d->d_k != d->d_v || !supported_d(d->d_k)) return GDN_ERR_UNSUPPORTED;
    const int64_t D = d->d_k;
    int64_t nt, a;
    if (!mul_ok(d->n, d->t, &nt)) return GDN_ERR_SHAPE;
    if (!mul_ok(nt, d->h_qk, &a) || !mul_ok(a, D, &s->qk)) return GDN_ERR_SHAPE;
    if (!mul_ok(nt, d->h_v, &s->gb) || !mul_ok(s->gb, D, &s->v)) return GDN_ERR_SHAPE;
    s->out = s->v;
    if (!mul_ok(d->n, d->h_v, &a) || !mul_ok(a, D * D, &s->state)) return GDN_ERR_SHAPE;
    // Keep every byte count (fp32 outputs are the largest) and grid size well inside range.
    const int64_t lim = INT64_C(1) << 60;
    if (s->out > lim / 4 || s->state > lim / 4 || s->qk > lim / 4) return GDN_ERR_SHAPE;
    if (d->n * (int64_t)d->h_v >= (INT64_C(1) << 31)) return GDN_ERR_SHAPE;
    if (d->t >= (INT64_C(1) << 40)) return GDN_ERR_SHAPE;
    s->esize = d->qkv_dtype == GDN_BF16 ? 2 : 4;
    return GDN_OK;
}

Range range_of(const void* p, int64_t elems, size_t esize)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, p ? lo + (uintptr_t)elems * esize : lo};
}

bool aligned(const void* p, uintptr_t a)
{
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

size_t workspace_for(const gdn_dims* d, int32_t chunk)
{
    if (d->t == 0 || d->n == 0) return 0;
    return chunk == 0 ? scan_workspace_bytes(d->n, d->t, d->h_qk, d->h_v, d->d_k)
                      : chunked_workspace_bytes(d->n, d->t, d->h_qk, d->h_v, d->d_k, chunk,
                                                d->qkv_dtype);
}

// Validate one call. mode: a chunk size (chunked), 0 (direct scan), -1 (decode, t == 1,
// no workspace) or -2 (no workspace and no method-specific limit: the whole of a segmented
// call, whose segments are validated again as they are issued).
gdn_status validate(const gdn_dims* d, int32_t mode, const void* q, const void* k,
                    const void* v, const float* g, const float* beta, const float* state_in,
                    float* out, float* state_out, void* ws, size_t ws_bytes, Call* call)
{
    Sizes s;
    gdn_status st = check_dims(d, &s);
    if (st != GDN_OK) return st;
    if (mode > 0 && !supported_chunk(mode)) return GDN_ERR_UNSUPPORTED;
    if (mode == -1 && d->t != 1) return GDN_ERR_SHAPE;
    // Every grid must fit in 31 bits: chunk workgroups (n * chunks * h_qk) and the scan's
    // normalisation rows (n * t * h_qk / 16).
    if (mode > 0 && d->n * ((d->t + mode - 1) / mode) * (int64_t)d->h_qk >= (INT64_C(1) << 31))
        return GDN_ERR_SHAPE;
    // The chunked kernels address one chunk of q, k, v and out with 32-bit byte offsets:
    // keep a chunk's extent (fp32 out is the largest) below 2^30 bytes.
    if (mode > 0 && (int64_t)mode * d->h_v * d->d_k * 4 + 64 >= (INT64_C(1) << 30))
        return GDN_ERR_SHAPE;
    if (mode == 0 && s.qk / d->d_k / 16 >= (INT64_C(1) << 31)) return GDN_ERR_SHAPE;

    const bool work = d->n > 0;
    const bool tokens = work && d->t > 0;
    if (work && !state_out) return GDN_ERR_NULL;
    if (tokens && (!q || !k || !v || !g || !beta || !out)) return GDN_ERR_NULL;

    const void* al16[] = {q, k, v, state_in, out, state_out, ws};
    for (const void* p : al16)
        if (p && !aligned(p, 16)) return GDN_ERR_ALIGN;
    if ((g && !aligned(g, 4)) || (beta && !aligned(beta, 4))) return GDN_ERR_ALIGN;

    size_t need = 0;
    if (mode >= 0 && tokens) need = workspace_for(d, mode);
    if (need > 0 && (!ws || ws_bytes < need)) return GDN_ERR_WORKSPACE;

    if (work) {
        const int64_t tq = tokens ? s.qk : 0, tv = tokens ? s.v : 0, tg = tokens ? s.gb : 0;
        const Range r_q = range_of(q, tq, s.esize), r_k = range_of(k, tq, s.esize);
        const Range r_v = range_of(v, tv, s.esize);
        const Range r_g = range_of(g, tg, 4), r_b = range_of(beta, tg, 4);
        const Range r_si = range_of(state_in, state_in ? s.state : 0, 4);
        const Range r_o = range_of(out, tv, 4), r_so = range_of(state_out, s.state, 4);
        const Range r_w = range_of(ws, (int64_t)need, 1);
        const Range inputs[] = {r_q, r_k, r_v, r_g, r_b};
        const Range outputs[] = {r_o, r_so, r_w};
        for (int i = 0; i < 3; ++i) {
            for (const Range& in : inputs)
                if (overlap(outputs[i], in)) return GDN_ERR_ALIAS;
            for (int j = i + 1; j < 3; ++j)
                if (overlap(outputs[i], outputs[j])) return GDN_ERR_ALIAS;
            // state_in may be state_out exactly (in place); any other overlap is an alias.
            if (overlap(outputs[i], r_si) && !(i == 1 && state_in == state_out))
                return GDN_ERR_ALIAS;
        }
    }

    *call = Call{d->n, d->t, d->h_qk, d->h_v, d->d_k, d->qkv_dtype, d->l2_eps,
                 q, k, v, g, beta, state_in, out, state_out, ws, ws_bytes, nullptr};
    return GDN_OK;
}

gdn_status finish(hipError_t e)
{
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// Copy (or zero) the state for an empty segment, t == 0.
__global__ void state_passthrough_kernel(const float4* __restrict__ src, float4* __restrict__ dst,
                                         int64_t n4)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

constexpr int32_t kMaxCalibBlocks = 1 << 20;

int32_t choose_chunk(const gdn_dims* d)
{
    int32_t pick = kCrossover[0].chunk;
    for (const auto& e : kCrossover)
        if (d->t >= e.min_t) pick = e.chunk;
    return pick;
}

// What gdn_prefill runs: kDecodeMethod for a single token (the decode step does the same
// arithmetic in one launch, with no workspace), else the table's choice (0 = direct scan).
constexpr int32_t kDecodeMethod = -1;
int32_t prefill_method(const gdn_dims* d)
{
    return d->t == 1 ? kDecodeMethod : choose_chunk(d);
}

size_t method_workspace(const gdn_dims* d, int32_t method)
{
    return method == kDecodeMethod ? 0 : workspace_for(d, method);
}

// ---------------------------------------------------------------- segmented prefill

// One segment of one sequence: a gdn_prefill call on sub-ranges of the whole call's buffers.
struct Piece {
    gdn_dims dims;
    const void *q, *k, *v;
    const float *g, *beta, *state_in;
    float *out, *state_out;
};

// Segment p of a call (sequence-major): tokens [t0, t0 + len) of sequence p / per_seq. The
// first segment of a sequence reads state_in; later ones continue from state_out in place.
struct SegmentPlan {
    const gdn_dims* d;
    int64_t seg_t, per_seq, pieces;
    const char *q, *k, *v;
    const float *g, *beta, *state_in;
    float *out, *state_out;

    SegmentPlan(const gdn_dims* d_, int64_t seg, const void* q_, const void* k_, const void* v_,
                const float* g_, const float* b_, const float* si, float* o, float* so)
        : d(d_), seg_t(seg), per_seq((d_->t + seg - 1) / seg), pieces(d_->n * per_seq),
          q(static_cast<const char*>(q_)), k(static_cast<const char*>(k_)),
          v(static_cast<const char*>(v_)), g(g_), beta(b_), state_in(si), out(o), state_out(so)
    {
    }

    Piece piece(int64_t p) const
    {
        const int64_t n = p / per_seq, t0 = (p % per_seq) * seg_t;
        const int64_t esz = d->qkv_dtype == GDN_BF16 ? 2 : 4;
        const int64_t row_qk = (int64_t)d->h_qk * d->d_k, row_v = (int64_t)d->h_v * d->d_v;
        const int64_t state_elems = (int64_t)d->h_v * d->d_k * d->d_v;
        const int64_t tok = n * d->t + t0;
        Piece x;
        x.dims = *d;
        x.dims.n = 1;
        x.dims.t = d->t - t0 < seg_t ? d->t - t0 : seg_t;
        x.q = q + tok * row_qk * esz;
        x.k = k + tok * row_qk * esz;
        x.v = v + tok * row_v * esz;
        x.g = g + tok * d->h_v;
        x.beta = beta + tok * d->h_v;
        x.state_in = t0 == 0 ? (state_in ? state_in + n * state_elems : nullptr)
                             : state_out + n * state_elems;
        x.out = out + tok * row_v;
        x.state_out = state_out + n * state_elems;
        return x;
    }
};

// The largest of a full segment's and the last segment's workspace, for one sequence.
size_t segment_workspace_bytes(const gdn_dims* d, int64_t seg_t)
{
    gdn_dims one = *d;
    one.n = 1;
    one.t = d->t < seg_t ? d->t : seg_t;
    size_t need = method_workspace(&one, prefill_method(&one));
    if (d->t % seg_t != 0 && d->t > seg_t) {
        one.t = d->t % seg_t;
        const size_t last = method_workspace(&one, prefill_method(&one));
        need = last > need ? last : need;
    }
    return need;
}

size_t slot_bytes(size_t b)
{
    return (b + 255) / 256 * 256;
}

// The side stream and events of the overlapped schedule: one set per device, created on
// first use and kept until the process ends. The stream has the default priority and does
// not synchronise with the null stream; every dependency is an explicit event wait.
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t start = nullptr, join = nullptr, prep[2] = {}, scan[2] = {};
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];
std::mutex g_side_mu;  // held while a call records into its device's events

gdn_status side_stream(SideStream** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
    SideStream& s = g_side[dev];
    if (!s.stream) {
        hipEvent_t* evs[] = {&s.start, &s.join, &s.prep[0], &s.prep[1], &s.scan[0], &s.scan[1]};
        for (hipEvent_t* e : evs)
            if (!*e && hipEventCreateWithFlags(e, hipEventDisableTiming) != hipSuccess)
                return GDN_ERR_HIP;
        if (hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) != hipSuccess) {
            s.stream = nullptr;
            return GDN_ERR_HIP;
        }
    }
    *out = &s;
    return GDN_OK;
}

// ---------------------------------------------------------------- allocation-free entry

// The workspace of gdn_prefill_segmented_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends. Host code never passes the array's name to a kernel
// (on the host it is only a stand-in symbol); it looks up each device's address once with
// hipGetSymbolAddress and passes that.
__device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

void* g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch`, looked up on the first call on that device.
gdn_status scratch_address(void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return GDN_ERR_HIP;
        }
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return GDN_OK;
}

}  // namespace

hipError_t launch_state_passthrough(const Call& c)
{
    if (c.state_in == c.state_out) return hipSuccess;
    const int64_t n4 = c.n * c.h_v * (int64_t)c.d * c.d / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(state_passthrough_kernel, dim3((unsigned)blocks), dim3(256), 0, c.stream,
                       reinterpret_cast<const float4*>(c.state_in),
                       reinterpret_cast<float4*>(c.state_out), n4);
    return hipGetLastError();
}

}  // namespace gdn

namespace gdn {
namespace {

// The checks gdn_prefill_segmented makes on the whole call, except those on the workspace:
// shapes, pointers, alignment, aliasing, and the method-specific limits of both segment
// lengths (seg_t and the remainder), all before anything is enqueued. *empty is set when
// there is nothing to do beyond the t == 0 state copy.
gdn_status check_segmented(const gdn_dims* d, int64_t seg_t, int32_t overlapped, const void* q,
                           const void* k, const void* v, const float* g, const float* beta,
                           const float* state_in, float* out, float* state_out)
{
    if (!d) return GDN_ERR_NULL;
    if (seg_t <= 0 || (overlapped != 0 && overlapped != 1)) return GDN_ERR_SHAPE;
    Call c;
    gdn_status st = validate(d, -2, q, k, v, g, beta, state_in, out, state_out, nullptr, 0, &c);
    if (st != GDN_OK || d->n == 0 || d->t == 0) return st;
    for (int64_t len : {d->t < seg_t ? d->t : seg_t, d->t % seg_t}) {
        if (len == 0) continue;
        gdn_dims one = *d;
        one.n = 1;
        one.t = len;
        st = validate(&one, prefill_method(&one), q, k, v, g, beta, state_in, out, state_out,
                      nullptr, 0, &c);
        if (st != GDN_OK && st != GDN_ERR_WORKSPACE) return st;
    }
    return GDN_OK;
}

// The in-order schedule: each segment as one gdn_prefill call on `stream`, all sharing ws.
gdn_status run_segments_in_order(const gdn_dims* d, int64_t seg_t, const void* q, const void* k,
                                 const void* v, const float* g, const float* beta,
                                 const float* state_in, float* out, float* state_out, void* ws,
                                 size_t ws_bytes, void* stream)
{
    const SegmentPlan plan(d, seg_t, q, k, v, g, beta, state_in, out, state_out);
    for (int64_t p = 0; p < plan.pieces; ++p) {
        const Piece x = plan.piece(p);
        const gdn_status st = gdn_prefill(&x.dims, x.q, x.k, x.v, x.g, x.beta, x.state_in,
                                          x.out, x.state_out, ws, ws_bytes, stream);
        if (st != GDN_OK) return st;
    }
    return GDN_OK;
}

}  // namespace
}  // namespace gdn

using namespace gdn;

extern "C" {

int32_t gdn_abi_version(void)
{
    return GDN_ABI_VERSION;
}

const char* gdn_status_str(int32_t s)
{
    switch (s) {
        case GDN_OK: return "GDN_OK: success";
        case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
        case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: invalid sizes or scalar arguments";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: head dim, chunk size or dtype not supported";
        case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: a pointer is misaligned";
        case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS: an output overlaps another buffer";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
        case GDN_ERR_HIP: return "GDN_ERR_HIP: the HIP runtime reported an error";
    }
    return "GDN_ERR_?: unknown status";
}

size_t gdn_workspace_bytes(const gdn_dims* d, int32_t chunk)
{
    Sizes s;
    if (check_dims(d, &s) != GDN_OK) return 0;
    if (chunk != 0 && !supported_chunk(chunk)) return 0;
    return workspace_for(d, chunk);
}

gdn_status gdn_prefill_chunked(const gdn_dims* d, int32_t chunk, const void* q, const void* k,
                               const void* v, const float* g, const float* beta,
                               const float* state_in, float* out, float* state_out,
                               void* ws, size_t ws_bytes, void* stream)
{
    if (d && !supported_chunk(chunk)) return GDN_ERR_UNSUPPORTED;
    Call c;
    gdn_status st = validate(d, chunk, q, k, v, g, beta, state_in, out, state_out, ws, ws_bytes, &c);
    if (st != GDN_OK) return st;
    if (c.n == 0) return GDN_OK;
    c.stream = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();  // report only errors raised by this call's launches
    return finish(c.t == 0 ? launch_state_passthrough(c) : launch_chunked(c, chunk));
}

gdn_status gdn_prefill_scan(const gdn_dims* d, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const float* state_in,
                            float* out, float* state_out, void* ws, size_t ws_bytes,
                            void* stream)
{
    Call c;
    gdn_status st = validate(d, 0, q, k, v, g, beta, state_in, out, state_out, ws, ws_bytes, &c);
    if (st != GDN_OK) return st;
    if (c.n == 0) return GDN_OK;
    c.stream = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return finish(c.t == 0 ? launch_state_passthrough(c) : launch_scan(c));
}

gdn_status gdn_prefill_scan_blockwise(const gdn_dims* d, int64_t block_t, const void* q,
                                      const void* k, const void* v, const float* g,
                                      const float* beta, const float* state_in, float* out,
                                      float* state_out, void* ws, size_t ws_bytes, void* stream)
{
    if (d && block_t <= 0) return GDN_ERR_SHAPE;
    Call c;
    gdn_status st = validate(d, 0, q, k, v, g, beta, state_in, out, state_out, ws, ws_bytes, &c);
    if (st != GDN_OK) return st;
    if (c.n == 0) return GDN_OK;
    c.stream = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return finish(c.t == 0 ? launch_state_passthrough(c) : launch_scan_blockwise(c, block_t));
}

gdn_status gdn_decode_step(const gdn_dims* d, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const float* state_in,
                           float* out, float* state_out, void* stream)
{
    Call c;
    gdn_status st = validate(d, -1, q, k, v, g, beta, state_in, out, state_out, nullptr, 0, &c);
    if (st != GDN_OK) return st;
    if (c.n == 0) return GDN_OK;
    c.stream = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return finish(launch_decode(c));
}

size_t gdn_prefill_segmented_workspace_bytes(const gdn_dims* d, int64_t seg_t, int32_t overlapped)
{
    Sizes s;
    if (seg_t <= 0 || (overlapped != 0 && overlapped != 1) || check_dims(d, &s) != GDN_OK ||
        d->n == 0 || d->t == 0)
        return 0;
    const size_t one = segment_workspace_bytes(d, seg_t);
    return overlapped ? 2 * slot_bytes(one) : one;
}

gdn_status gdn_prefill_segmented(const gdn_dims* d, int64_t seg_t, int32_t overlapped,
                                 const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* state_in, float* out,
                                 float* state_out, void* ws, size_t ws_bytes, void* stream)
{
    // The whole call is validated as one (shapes, pointers, alignment, aliasing, both
    // segment lengths' limits); every segment call below is a sub-range of it.
    gdn_status st = check_segmented(d, seg_t, overlapped, q, k, v, g, beta, state_in, out,
                                    state_out);
    if (st != GDN_OK) return st;
    if (d->n == 0) return GDN_OK;
    if (d->t == 0) return gdn_prefill(d, q, k, v, g, beta, state_in, out, state_out, ws, ws_bytes, stream);
    const size_t need = gdn_prefill_segmented_workspace_bytes(d, seg_t, overlapped);
    if (need > 0 && (!ws || ws_bytes < need)) return GDN_ERR_WORKSPACE;
    if (ws && need > 0) {
        // the workspace must not overlap any buffer of the call
        Sizes s;
        check_dims(d, &s);
        const Range r_w = range_of(ws, (int64_t)need, 1);
        const Range others[] = {range_of(q, s.qk, s.esize), range_of(k, s.qk, s.esize),
                                range_of(v, s.v, s.esize), range_of(g, s.gb, 4),
                                range_of(beta, s.gb, 4), range_of(out, s.v, 4),
                                range_of(state_out, s.state, 4),
                                range_of(state_in, state_in ? s.state : 0, 4)};
        for (const Range& r : others)
            if (overlap(r_w, r)) return GDN_ERR_ALIAS;
        if (!aligned(ws, 16)) return GDN_ERR_ALIGN;
    }
    if (!overlapped)
        return run_segments_in_order(d, seg_t, q, k, v, g, beta, state_in, out, state_out, ws,
                                     ws_bytes, stream);

    Call c;
    const SegmentPlan plan(d, seg_t, q, k, v, g, beta, state_in, out, state_out);

    // Overlapped: the per-chunk preparation of segment p + 1 runs on the side stream while
    // the sequential pass of segment p runs on the caller's stream, with the workspace split
    // into two slots used by alternate segments.
    hipStream_t main_s = static_cast<hipStream_t>(stream);
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(main_s, &cap) != hipSuccess) return GDN_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone) return GDN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream* side = nullptr;
    st = side_stream(&side);
    if (st != GDN_OK) return st;
    const size_t slot = slot_bytes(segment_workspace_bytes(d, seg_t));
    (void)hipGetLastError();
    hipError_t e = hipEventRecord(side->start, main_s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->start, 0);
    for (int64_t p = 0; p < plan.pieces && e == hipSuccess; ++p) {
        const Piece x = plan.piece(p);
        const int sl = (int)(p & 1);
        void* wsp = static_cast<char*>(ws) + sl * slot;
        const int32_t chunk = prefill_method(&x.dims);
        st = validate(&x.dims, chunk, x.q, x.k, x.v, x.g, x.beta, x.state_in, x.out,
                      x.state_out, wsp, slot, &c);
        if (st != GDN_OK) break;
        if (chunk == kDecodeMethod) {
            c.stream = main_s;
            e = launch_decode(c);
        } else if (chunk > 0) {
            // the slot's previous user (segment p - 2) has finished its sequential pass
            if (p >= 2) e = hipStreamWaitEvent(side->stream, side->scan[sl], 0);
            c.stream = side->stream;
            if (e == hipSuccess) e = launch_chunked(c, chunk, kChunkPrep);
            if (e == hipSuccess) e = hipEventRecord(side->prep[sl], side->stream);
            if (e == hipSuccess) e = hipStreamWaitEvent(main_s, side->prep[sl], 0);
            c.stream = main_s;
            if (e == hipSuccess) e = launch_chunked(c, chunk, kChunkScan);
        } else {
            c.stream = main_s;
            e = launch_scan(c);
        }
        if (e == hipSuccess) e = hipEventRecord(side->scan[sl], main_s);
    }
    // The caller's stream orders after everything enqueued on the side stream, also when
    // the loop stopped early.
    hipError_t j = hipEventRecord(side->join, side->stream);
    if (j == hipSuccess) j = hipStreamWaitEvent(main_s, side->join, 0);
    if (st != GDN_OK) return st;
    return finish(e != hipSuccess ? e : j);
}

size_t gdn_noalloc_scratch_bytes(void)
{
    return GDN_NOALLOC_SCRATCH_BYTES;
}

gdn_status gdn_prefill_segmented_noalloc(const gdn_dims* d, int64_t seg_t, const void* q,
                                         const void* k, const void* v, const float* g,
                                         const float* beta, const float* state_in, float* out,
                                         float* state_out, void* stream)
{
    gdn_status st = check_segmented(d, seg_t, 0, q, k, v, g, beta, state_in, out, state_out);
    if (st != GDN_OK) return st;
    if (d->n == 0) return GDN_OK;
    const size_t need = d->t == 0 ? 0 : gdn_prefill_segmented_workspace_bytes(d, seg_t, 0);
    if (need > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        st = scratch_address(&ws);
        if (st != GDN_OK) return st;
    }
    return run_segments_in_order(d, seg_t, q, k, v, g, beta, state_in, out, state_out, ws,
                                 need > 0 ? (size_t)GDN_NOALLOC_SCRATCH_BYTES : 0, stream);
}

gdn_status gdn_decode_graph_create(const gdn_dims* d, int32_t layers, const void* const* q,
                                   const void* const* k, const void* const* v,
                                   const float* const* g, const float* const* beta,
                                   float* const* state, float* const* out, void* stream,
                                   gdn_graph* graph)
{
    if (!graph) return GDN_ERR_NULL;
    *graph = nullptr;
    if (!d || !q || !k || !v || !g || !beta || !state || !out || !stream) return GDN_ERR_NULL;
    if (layers < 0) return GDN_ERR_SHAPE;
    // Every layer is validated before anything is recorded.
    std::vector<Call> calls((size_t)layers);
    for (int32_t i = 0; i < layers; ++i) {
        gdn_status st = validate(d, -1, q[i], k[i], v[i], g[i], beta[i], state[i], out[i],
                                 state[i], nullptr, 0, &calls[(size_t)i]);
        if (st != GDN_OK) return st;
        calls[(size_t)i].stream = static_cast<hipStream_t>(stream);
    }
    (void)hipGetLastError();
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) return GDN_ERR_HIP;
    hipError_t launch_err = hipSuccess;
    for (const Call& c : calls)
        if (c.n > 0 && launch_err == hipSuccess) launch_err = launch_decode(c);
    hipGraph_t g_rec = nullptr;
    const hipError_t end_err = hipStreamEndCapture(s, &g_rec);
    if (launch_err != hipSuccess || end_err != hipSuccess || !g_rec) {
        if (g_rec) (void)hipGraphDestroy(g_rec);
        (void)hipGetLastError();
        return GDN_ERR_HIP;
    }
    hipGraphExec_t exec = nullptr;
    const hipError_t inst_err = hipGraphInstantiate(&exec, g_rec, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g_rec);
    if (inst_err != hipSuccess || !exec) {
        (void)hipGetLastError();
        return GDN_ERR_HIP;
    }
    *graph = new gdn_graph_rec{exec};
    return GDN_OK;
}

gdn_status gdn_graph_launch(gdn_graph graph, void* stream)
{
    if (!graph) return GDN_ERR_NULL;
    (void)hipGetLastError();
    return finish(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_graph_destroy(gdn_graph graph)
{
    if (!graph) return GDN_OK;
    const hipError_t e = hipGraphExecDestroy(graph->exec);
    delete graph;
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_prefill_choose(const gdn_dims* d, int32_t* chunk_or_zero)
{
    Sizes s;
    if (!chunk_or_zero) return GDN_ERR_NULL;
    gdn_status st = check_dims(d, &s);
    if (st != GDN_OK) return st;
    *chunk_or_zero = choose_chunk(d);
    return GDN_OK;
}

size_t gdn_prefill_workspace_bytes(const gdn_dims* d)
{
    Sizes s;
    if (check_dims(d, &s) != GDN_OK) return 0;
    return method_workspace(d, prefill_method(d));
}

gdn_status gdn_prefill(const gdn_dims* d, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const float* state_in, float* out,
                       float* state_out, void* ws, size_t ws_bytes, void* stream)
{
    int32_t chunk = 0;
    gdn_status st = gdn_prefill_choose(d, &chunk);
    if (st != GDN_OK) return st;
    if (d->t == 1) return gdn_decode_step(d, q, k, v, g, beta, state_in, out, state_out, stream);
    return chunk == 0 ? gdn_prefill_scan(d, q, k, v, g, beta, state_in, out, state_out, ws,
                                         ws_bytes, stream)
                      : gdn_prefill_chunked(d, chunk, q, k, v, g, beta, state_in, out,
                                            state_out, ws, ws_bytes, stream);
}

int64_t gdn_calib_mfma_bf16_flops(int64_t iters, int32_t blocks)
{
    if (iters <= 0 || blocks <= 0 || blocks > kMaxCalibBlocks) return 0;
    // 4 waves per workgroup, 4 MFMAs per iteration, 32 x 32 x 16 multiply-adds each
    return (int64_t)blocks * 4 * iters * 4 * (32 * 32 * 16 * 2);
}

gdn_status gdn_calib_mfma_bf16(int64_t iters, int32_t blocks, float* sink, void* stream)
{
    if (!sink) return GDN_ERR_NULL;
    if (iters <= 0 || blocks <= 0 || blocks > kMaxCalibBlocks) return GDN_ERR_SHAPE;
    if (!aligned(sink, 4)) return GDN_ERR_ALIGN;
    (void)hipGetLastError();
    return finish(launch_mfma_loop(iters, blocks, sink, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_calib_stream_copy(const void* src, void* dst, int64_t bytes, int32_t blocks,
                                 void* stream)
{
    if (!src || !dst) return GDN_ERR_NULL;
    if (bytes <= 0 || bytes % 16 != 0 || blocks <= 0 || blocks > kMaxCalibBlocks)
        return GDN_ERR_SHAPE;
    if (!aligned(src, 16) || !aligned(dst, 16)) return GDN_ERR_ALIGN;
    const Range a = range_of(src, bytes, 1), b = range_of(dst, bytes, 1);
    if (overlap(a, b)) return GDN_ERR_ALIAS;
    (void)hipGetLastError();
    return finish(launch_stream_copy(src, dst, bytes / 16, blocks, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_debug_fill_lds(uint32_t pattern, int32_t blocks, uint32_t* sink, void* stream)
{
    if (!sink) return GDN_ERR_NULL;
    if (blocks <= 0 || blocks > kMaxCalibBlocks) return GDN_ERR_SHAPE;
    if (!aligned(sink, 4)) return GDN_ERR_ALIGN;
    (void)hipGetLastError();
    return finish(launch_lds_fill(pattern, blocks, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
