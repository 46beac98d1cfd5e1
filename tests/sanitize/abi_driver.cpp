// Drives the host-side validation of libgdn's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point with bad arguments (NULL, shapes, alignment,
// aliasing, workspace), the size queries and the status strings. The device addresses are
// fake and never dereferenced: every case returns before the first HIP call. Exits non-zero
// on an unexpected return value.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "gdn.h"

namespace {

int failures = 0;

void expect(const char* what, long got, long want)
{
    if (got != want) {
        std::printf("FAIL %s: got %ld, want %ld\n", what, got, want);
        ++failures;
    }
}

// Fake, page-separated device buffers of a call with the given shape.
struct Bufs {
    gdn_dims d;
    uintptr_t q, k, v, g, beta, si, out, so, ws;
    Bufs(int64_t n, int64_t t, int32_t h_qk, int32_t h_v, int32_t dk)
    {
        d = gdn_dims{n, t, h_qk, h_v, dk, dk, GDN_BF16, 1e-6f};
        uintptr_t base = 0x7F0000000000ull;
        auto take = [&](uint64_t bytes) {
            const uintptr_t a = base;
            base += (bytes + 4095) / 4096 * 4096 + 4096;
            return a;
        };
        q = take(n * t * h_qk * dk * 2);
        k = take(n * t * h_qk * dk * 2);
        v = take(n * t * h_v * dk * 2);
        g = take(n * t * h_v * 4);
        beta = take(n * t * h_v * 4);
        si = take(n * h_v * dk * dk * 4);
        out = take(n * t * h_v * dk * 4);
        so = take(n * h_v * dk * dk * 4);
        ws = take(64ull << 20);
    }
};

template <typename T>
T* P(uintptr_t a)
{
    return reinterpret_cast<T*>(a);
}

}  // namespace

int main()
{
    const size_t WS = 64ull << 20;
    Bufs b(1, 64, 2, 4, 32);
    const void* vq = P<void>(b.q);
    const void* vk = P<void>(b.k);
    const void* vv = P<void>(b.v);
    const float* g = P<float>(b.g);
    const float* be = P<float>(b.beta);
    const float* si = P<float>(b.si);
    float* out = P<float>(b.out);
    float* so = P<float>(b.so);
    void* ws = P<void>(b.ws);

    // chunked
    expect("chunked null dims", gdn_prefill_chunked(nullptr, 32, vq, vk, vv, g, be, si, out, so, ws, WS, nullptr), GDN_ERR_NULL);
    expect("chunked bad chunk", gdn_prefill_chunked(&b.d, 48, vq, vk, vv, g, be, si, out, so, ws, WS, nullptr), GDN_ERR_UNSUPPORTED);
    expect("chunked null q", gdn_prefill_chunked(&b.d, 32, nullptr, vk, vv, g, be, si, out, so, ws, WS, nullptr), GDN_ERR_NULL);
    expect("chunked misaligned out", gdn_prefill_chunked(&b.d, 32, vq, vk, vv, g, be, si, P<float>(b.out + 4), so, ws, WS, nullptr), GDN_ERR_ALIGN);
    expect("chunked out aliases q", gdn_prefill_chunked(&b.d, 32, vq, vk, vv, g, be, si, P<float>(b.q), so, ws, WS, nullptr), GDN_ERR_ALIAS);
    expect("chunked short workspace", gdn_prefill_chunked(&b.d, 32, vq, vk, vv, g, be, si, out, so, ws, 16, nullptr), GDN_ERR_WORKSPACE);
    expect("chunked workspace aliases state", gdn_prefill_chunked(&b.d, 32, vq, vk, vv, g, be, si, out, so, P<void>(b.so), WS, nullptr), GDN_ERR_ALIAS);
    gdn_dims bad = b.d;
    bad.h_v = 3;
    expect("chunked h_v % h_qk", gdn_prefill_chunked(&bad, 32, vq, vk, vv, g, be, si, out, so, ws, WS, nullptr), GDN_ERR_SHAPE);
    bad = b.d;
    bad.d_k = bad.d_v = 40;
    expect("chunked d 40", gdn_prefill_chunked(&bad, 32, vq, vk, vv, g, be, si, out, so, ws, WS, nullptr), GDN_ERR_UNSUPPORTED);
    bad = b.d;
    bad.t = -1;
    expect("chunked t < 0", gdn_prefill_chunked(&bad, 32, vq, vk, vv, g, be, si, out, so, ws, WS, nullptr), GDN_ERR_SHAPE);
    bad = b.d;
    bad.n = INT64_MAX / 4;
    expect("chunked size overflow", gdn_prefill_chunked(&bad, 32, vq, vk, vv, g, be, si, out, so, ws, WS, nullptr), GDN_ERR_SHAPE);
    bad = b.d;
    bad.l2_eps = -1.0f;
    expect("chunked eps < 0", gdn_prefill_chunked(&bad, 32, vq, vk, vv, g, be, si, out, so, ws, WS, nullptr), GDN_ERR_SHAPE);

    // scan, blockwise scan, choice, decode
    expect("scan null state_out", gdn_prefill_scan(&b.d, vq, vk, vv, g, be, si, out, nullptr, ws, WS, nullptr), GDN_ERR_NULL);
    expect("blockwise block 0", gdn_prefill_scan_blockwise(&b.d, 0, vq, vk, vv, g, be, si, out, so, ws, WS, nullptr), GDN_ERR_SHAPE);
    expect("blockwise alias", gdn_prefill_scan_blockwise(&b.d, 8, vq, vk, vv, g, be, si, P<float>(b.v), so, ws, WS, nullptr), GDN_ERR_ALIAS);
    expect("prefill null", gdn_prefill(&b.d, vq, vk, vv, g, be, si, out, so, nullptr, 0, nullptr), GDN_ERR_WORKSPACE);
    int32_t chunk = -1;
    expect("choose", gdn_prefill_choose(&b.d, &chunk), GDN_OK);
    expect("choose null", gdn_prefill_choose(&b.d, nullptr), GDN_ERR_NULL);
    Bufs one(30, 1, 16, 32, 128);
    gdn_dims two = one.d;
    two.t = 2;
    expect("decode t 2", gdn_decode_step(&two, P<void>(one.q), P<void>(one.k), P<void>(one.v), P<float>(one.g), P<float>(one.beta), P<float>(one.si), P<float>(one.out), P<float>(one.so), nullptr), GDN_ERR_SHAPE);
    expect("decode alias", gdn_decode_step(&one.d, P<void>(one.q), P<void>(one.k), P<void>(one.v), P<float>(one.g), P<float>(one.beta), P<float>(one.si), P<float>(one.si + 64), P<float>(one.so), nullptr), GDN_ERR_ALIAS);

    // segmented (64-token segments: the chunked path, which needs a workspace)
    expect("segmented seg 0", gdn_prefill_segmented(&b.d, 0, 0, vq, vk, vv, g, be, si, out, so, ws, WS, nullptr), GDN_ERR_SHAPE);
    expect("segmented overlapped 2", gdn_prefill_segmented(&b.d, 64, 2, vq, vk, vv, g, be, si, out, so, ws, WS, nullptr), GDN_ERR_SHAPE);
    expect("segmented short workspace", gdn_prefill_segmented(&b.d, 64, 1, vq, vk, vv, g, be, si, out, so, ws, 16, nullptr), GDN_ERR_WORKSPACE);
    expect("segmented misaligned workspace", gdn_prefill_segmented(&b.d, 64, 1, vq, vk, vv, g, be, si, out, so, P<void>(b.ws + 8), WS, nullptr), GDN_ERR_ALIGN);

    // decode graph (checked before any recording)
    const void* qs[1] = {P<void>(one.q)};
    const void* ks[1] = {P<void>(one.k)};
    const void* vs[1] = {P<void>(one.v)};
    const float* gs[1] = {P<float>(one.g)};
    const float* bs[1] = {P<float>(one.beta)};
    float* sts[1] = {P<float>(one.si)};
    float* outs[1] = {P<float>(one.out)};
    gdn_graph h = nullptr;
    expect("graph null stream", gdn_decode_graph_create(&one.d, 1, qs, ks, vs, gs, bs, sts, outs, nullptr, &h), GDN_ERR_NULL);
    expect("graph null handle", gdn_decode_graph_create(&one.d, 1, qs, ks, vs, gs, bs, sts, outs, reinterpret_cast<void*>(0x1000), nullptr), GDN_ERR_NULL);
    expect("graph destroy null", gdn_graph_destroy(nullptr), GDN_OK);
    expect("graph launch null", gdn_graph_launch(nullptr, nullptr), GDN_ERR_NULL);

    // calibration loop arguments
    expect("calib null", gdn_calib_mfma_bf16(10, 4, nullptr, nullptr), GDN_ERR_NULL);
    expect("calib iters", gdn_calib_mfma_bf16(0, 4, P<float>(b.out), nullptr), GDN_ERR_SHAPE);

    // size queries and strings
    expect("workspace > 0", gdn_workspace_bytes(&b.d, 32) > 0, 1);
    expect("workspace bad chunk", (long)gdn_workspace_bytes(&b.d, 48), 0);
    expect("segmented workspace", gdn_prefill_segmented_workspace_bytes(&b.d, 16, 1) >= 2 * gdn_prefill_segmented_workspace_bytes(&b.d, 16, 0), 1);
    for (int s = -1; s <= 8; ++s) {
        const char* str = gdn_status_str(s);
        expect("status string", str != nullptr && std::strlen(str) > 0, 1);
    }
    expect("abi version", gdn_abi_version(), GDN_ABI_VERSION);

    std::printf("abi driver %s (%d failures)\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
