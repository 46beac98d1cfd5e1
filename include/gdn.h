/*
 * gdn.h -- C ABI of libgdn.so: the Gated DeltaNet layer recurrence on AMD Instinct
 * MI355X (gfx950), prefill and batch-1 decode.
 *
 * Source of the operation: "Optimizing on-device inference for Apple Silicon"
 * (Perplexity, 2026).
 *   - Section "Qwen creates three distinct workload shapes": each Gated DeltaNet layer
 *     keeps a fixed-size recurrent state; a learned gate decides how much of the old
 *     state to keep and a delta update writes the current token in; every token depends
 *     on the state after the previous token. Prefill may either scan the tokens directly
 *     or re-block the updates into chunks that expose matrix work; which is faster depends
 *     on the model dimensions, the workload and the hardware.
 *   - Section "Keep the recurrent state on-chip": the state and its gate are 32-bit
 *     floats (rounding compounds over sequential updates); queries and keys stay bf16;
 *     the state is loaded once, carried through the scan and written back once.
 *   - Section "Bound temporary memory with prompt chunking": a long prompt runs as
 *     bounded segments whose recurrent state carries the context forward, without
 *     changing the result. Here: pass one call's state_out as the next call's state_in.
 *   - Section "Decode: minimise bytes moved per token" and its fused-chain list: decode
 *     is bound by bytes moved per token; the recurrent update is fused with its
 *     normalisation (here: the L2 normalisation of q and k).
 *
 * The recurrence (the gated delta rule; the page states it only in words). Per sequence,
 * per V head h, for tokens t = 1..T:
 *
 *     S_t = exp(g_t) * S_{t-1} * (I - beta_t * khat_t * khat_t^T) + beta_t * v_t * khat_t^T
 *     o_t = S_t * qhat_t                     (the state after token t's own update)
 *
 * with S_t of shape d_v x d_k, qhat = q / sqrt(sum(q^2) + l2_eps) and likewise khat, per
 * token and QK head, and V head h reading QK head h / (h_v / h_qk) (consecutive V heads
 * share a QK head). No 1/sqrt(d_k) query scale is applied; o is linear in q, so a caller
 * that wants one scales `out`.
 *
 * Layouts. Every tensor is dense, row-major (C order), with no padding:
 *   q, k        [n][t][h_qk][d_k]   qkv_dtype (bf16 or fp32)
 *   v           [n][t][h_v][d_v]    qkv_dtype
 *   g, beta     [n][t][h_v]         fp32; g is the log of the per-token decay (exp(g) is
 *                                   applied), beta the write strength. Neither is clamped.
 *   state_in,   [n][h_v][d_k][d_v]  fp32; element [i][j] holds S[j][i] (the state is stored
 *   state_out                        transposed, d_k-major, so a value channel j is a
 *                                   strided column and a key row i is contiguous)
 *   out         [n][t][h_v][d_v]    fp32
 * n counts independent sequences; for the stacked decode step it counts layers.
 *
 * Pointers and ownership. Every data pointer is a DEVICE pointer on the current HIP
 * device. The caller allocates and owns every buffer, including the workspace. The
 * library never allocates device memory, frees or synchronises, and is safe to call from
 * several host threads, with two exceptions that hold runtime objects: the decode graph
 * handle (gdn_decode_graph_create owns the HIP graph it records until
 * gdn_graph_destroy), and the overlapped schedule of gdn_prefill_segmented, which creates
 * one side stream and a few events per device on first use, keeps them until the process
 * ends, and serialises the calls that enqueue on them. Every compute call only enqueues
 * kernels on `stream` (a hipStream_t; NULL is the default stream) and returns; results are
 * ready when the stream reaches that point. The compute calls make no memset or copy
 * calls, so they may be recorded under HIP stream capture (except the overlapped
 * segmented schedule, which refuses a capturing stream).
 *
 * Alignment. q, k, v, state_in, state_out, out and workspace must be 16-byte aligned;
 * g and beta 4-byte aligned.
 *
 * Aliasing. state_in == state_out is allowed (update in place). Any other overlap of an
 * output (out, state_out, workspace) with any other buffer is GDN_ERR_ALIAS. Inputs may
 * overlap each other (for example q == k).
 *
 * Errors. All arguments are validated on the host before any HIP call. On any error
 * nothing is enqueued and out/state_out are untouched. A launch failure reported by
 * hipGetLastError returns GDN_ERR_HIP. Faults inside a kernel surface at the caller's next
 * stream synchronisation, as for any HIP kernel.
 *
 * Supported: d_k == d_v in {16, 32, 64, 128}; chunk in {16, 32, 64, 128}; h_v a multiple
 * of h_qk; n >= 0 (n == 0 is a no-op); t >= 0 for prefill (t == 0 copies state_in to
 * state_out, or zeroes state_out when state_in is NULL); t == 1 for decode.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 2

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,        /* a required pointer is NULL                               */
    GDN_ERR_SHAPE = 2,       /* negative or inconsistent sizes, size overflow            */
    GDN_ERR_UNSUPPORTED = 3, /* valid but not built: head dim, chunk size, dtype          */
    GDN_ERR_ALIGN = 4,       /* pointer misaligned                                       */
    GDN_ERR_ALIAS = 5,       /* an output overlaps another buffer (see Aliasing)          */
    GDN_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than gdn_workspace_bytes()      */
    GDN_ERR_HIP = 7          /* the HIP runtime reported an error at launch               */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef struct {
    int64_t n;         /* independent sequences (or stacked layers for decode)     */
    int64_t t;         /* tokens in this call                                      */
    int32_t h_qk;      /* query/key heads                                          */
    int32_t h_v;       /* value heads, a multiple of h_qk                          */
    int32_t d_k;       /* key head dimension                                       */
    int32_t d_v;       /* value head dimension (must equal d_k)                    */
    int32_t qkv_dtype; /* gdn_dtype of q, k and v                                  */
    float l2_eps;      /* added to sum(x^2) under the square root; 1e-6 is typical */
} gdn_dims;

/* Version of this header the library was built from (GDN_ABI_VERSION). */
int32_t gdn_abi_version(void);

/* Static string for a status code (any int32_t: a value that is no gdn_status gives an
 * "unknown status" string); never NULL. */
const char* gdn_status_str(int32_t status);

/*
 * Workspace bytes a call needs: chunk in {16,32,64,128} for gdn_prefill_chunked, chunk 0
 * for gdn_prefill_scan (always 0: the direct scan needs none). Returns 0 for invalid or
 * unsupported dims (and for t == 0). gdn_decode_step needs no workspace.
 */
size_t gdn_workspace_bytes(const gdn_dims* dims, int32_t chunk);

/*
 * Chunked prefill: the recurrence re-blocked into chunks of `chunk` tokens (the chunked
 * evaluation of "Qwen creates three distinct workload shapes"). Within a chunk the
 * updates are solved jointly (UT transform of the delta-rule updates, WY form) with bf16
 * matrix-core products; the state is carried across chunks on chip. t need not be a
 * multiple of chunk. Needs gdn_workspace_bytes(dims, chunk) bytes of workspace.
 * GDN_ERR_SHAPE also when chunk * h_v * d_v * 4 + 64 >= 2^30 (one chunk's output rows
 * must fit 32-bit in-kernel offsets).
 */
gdn_status gdn_prefill_chunked(const gdn_dims* dims, int32_t chunk, const void* q,
                               const void* k, const void* v, const float* g,
                               const float* beta, const float* state_in, float* out,
                               float* state_out, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Direct-scan prefill: tokens in order, the state held in registers for the whole call
 * and written back once ("Keep the recurrent state on-chip"). The inputs are staged and
 * normalised on chip, so it needs no workspace (gdn_workspace_bytes(dims, 0) is 0; the
 * workspace arguments are ignored).
 */
gdn_status gdn_prefill_scan(const gdn_dims* dims, const void* q, const void* k,
                            const void* v, const float* g, const float* beta,
                            const float* state_in, float* out, float* state_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * The residency ablation of the direct scan ("Keep the recurrent state on-chip": with the
 * state not kept resident, a blockwise scan moves the whole state through device memory
 * over and over; the pages count the bytes per layer for a 2K-token prompt). Same
 * arithmetic as gdn_prefill_scan, and the same bits: the scan kernel runs once per block of
 * block_t tokens of each sequence (normalising that block's q/k rows on chip), reading the
 * state at the start of the block (state_in for the first block, else state_out) and
 * writing it to state_out at the end, so each block moves 2 x h_v x d_k x d_v x 4 bytes of
 * state per sequence. n x ceil(t / block_t) scan launches on `stream`. Workspace and
 * errors as for gdn_prefill_scan; GDN_ERR_SHAPE for block_t <= 0. For measurement, not for
 * speed.
 */
gdn_status gdn_prefill_scan_blockwise(const gdn_dims* dims, int64_t block_t, const void* q,
                                      const void* k, const void* v, const float* g,
                                      const float* beta, const float* state_in, float* out,
                                      float* state_out, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * Batch-1 decode step (dims->t must be 1): one token per sequence; each (sequence, V
 * head) state streams from HBM through registers back to HBM once, with the q/k
 * normalisation fused in. No workspace.
 * Source: "Decode: minimise bytes moved per token" -- at batch 1 a decode step is bound by
 * the bytes it moves per token, and the fused-chain list there pairs the recurrent update
 * with its normalisation; the per-token update itself is the one of "Qwen creates three
 * distinct workload shapes" (every token depends on the state after the previous one).
 */
gdn_status gdn_decode_step(const gdn_dims* dims, const void* q, const void* k,
                           const void* v, const float* g, const float* beta,
                           const float* state_in, float* out, float* state_out,
                           void* stream);

/*
 * Decode graph: one decode token through `layers` stacked GDN layers as dependent
 * per-layer steps, recorded once as a HIP graph and replayed per token ("Decode: minimise
 * bytes moved per token": keep each decode step on the GPU with as little host work per
 * token as possible). Layer i runs gdn_decode_step(dims, q[i], k[i], v[i], g[i], beta[i],
 * state[i], out[i], state[i]) -- its state updated in place -- after layer i - 1, in one
 * stream. dims (t == 1, the same for every layer) and the pointer arrays (host arrays of
 * `layers` device pointers) are validated per layer as for gdn_decode_step before anything
 * is recorded; the device pointers are fixed in the graph, so the caller writes each
 * token's inputs into the same buffers and keeps them alive until gdn_graph_destroy.
 * `stream` must be a non-NULL stream (the legacy default stream cannot be captured); it is
 * used only while recording. *graph receives the handle (NULL on error). Errors:
 * GDN_ERR_NULL (a NULL pointer or stream), the gdn_decode_step errors of any layer
 * (checked before recording), GDN_ERR_HIP if recording or instantiation fails.
 *
 * gdn_graph_launch enqueues one replay (all layers) on `stream` (NULL allowed);
 * gdn_graph_destroy releases the handle (NULL is a no-op). Replays of one handle that
 * overlap in time race on its buffers, as any two calls on the same buffers would.
 */
typedef struct gdn_graph_rec* gdn_graph;

gdn_status gdn_decode_graph_create(const gdn_dims* dims, int32_t layers,
                                   const void* const* q, const void* const* k,
                                   const void* const* v, const float* const* g,
                                   const float* const* beta, float* const* state,
                                   float* const* out, void* stream, gdn_graph* graph);
gdn_status gdn_graph_launch(gdn_graph graph, void* stream);
gdn_status gdn_graph_destroy(gdn_graph graph);

/*
 * Prefill method for these dims, from the measured scan-versus-chunk crossover on
 * MI355X: *chunk_or_zero receives 0 for the direct scan or the chunk size to pass to
 * gdn_prefill_chunked.
 * Source: "Qwen creates three distinct workload shapes" -- the direct scan and the chunked
 * form compute the same result, and which one is faster depends on the model dimensions,
 * the workload and the hardware, so the choice is measured rather than fixed ("Optimization
 * strategy": decide from measurements on the target machine).
 * Scope of the table: it was measured for one sequence (n = 1), 16 QK / 32 V heads,
 * d = 128 and bf16 q/k/v, and is keyed on the token count only; other head counts, head
 * dimensions, fp32 inputs and batched calls get the same pick by length, which is correct
 * (every method computes the same result) but not tuned for them.
 */
gdn_status gdn_prefill_choose(const gdn_dims* dims, int32_t* chunk_or_zero);

/*
 * Prefill with the method gdn_prefill_choose picks, except that a single token (t == 1)
 * runs as gdn_decode_step (the same arithmetic in one launch, no workspace). The workspace
 * must be at least gdn_prefill_workspace_bytes(dims): gdn_workspace_bytes(dims, chosen
 * chunk), or 0 when t == 1.
 */
size_t gdn_prefill_workspace_bytes(const gdn_dims* dims);
gdn_status gdn_prefill(const gdn_dims* dims, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const float* state_in,
                       float* out, float* state_out, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Segmented prefill ("Bound temporary memory with prompt chunking": a long prompt runs as
 * bounded segments whose recurrent state carries the context forward, without changing
 * the result). Each sequence's tokens are taken in consecutive segments of seg_t tokens
 * (the last may be shorter); each segment runs the method gdn_prefill runs for its
 * length, on one sequence, with the state carried from segment to segment through
 * state_out (updated in place after the first segment, which reads state_in). The
 * workspace is reused by every segment, so its size depends on seg_t, not on t:
 * gdn_prefill_segmented_workspace_bytes(dims, seg_t, overlapped). seg_t must be
 * positive; the results agree with gdn_prefill to within rounding (the chunk boundaries
 * restart at each segment), and are the same bits with overlapped 0 or 1.
 *
 * overlapped = 0: the segments run one after another on `stream`.
 * overlapped = 1: the workspace holds two segment slots (twice the bytes, each slot
 *   rounded up to 256). The per-chunk preparation of a chunked segment runs on a second
 *   stream that the library creates on first use (one per device, default priority, kept
 *   until the process ends) while the previous segment's sequential pass runs on
 *   `stream`; events order the two, and `stream` waits for all of the call's work before
 *   anything enqueued after it. The current device must be the device of `stream`. Calls
 *   on one device are serialised on the host while they enqueue. Not for graph capture:
 *   GDN_ERR_UNSUPPORTED when `stream` is capturing.
 *
 * Errors as for gdn_prefill on the whole call, checked before anything is enqueued
 * (including the method limits of both segment lengths); GDN_ERR_SHAPE for seg_t <= 0 or
 * overlapped not 0 or 1; GDN_ERR_HIP if the runtime fails to create or record the side
 * stream's events. gdn_prefill_segmented_workspace_bytes returns 0 for an empty call or
 * invalid arguments.
 */
size_t gdn_prefill_segmented_workspace_bytes(const gdn_dims* dims, int64_t seg_t,
                                             int32_t overlapped);
gdn_status gdn_prefill_segmented(const gdn_dims* dims, int64_t seg_t, int32_t overlapped,
                                 const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* state_in, float* out,
                                 float* state_out, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Allocation-free segmented prefill, for callers that cannot allocate device memory: code
 * recorded under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Computes exactly what gdn_prefill_segmented(dims, seg_t, 0, ...) computes (the in-order
 * schedule, the same kernels, the same bits), but takes no workspace argument: the
 * segments' workspace is a static device array inside the library of
 * GDN_NOALLOC_SCRATCH_BYTES bytes per GPU, reserved when the library's code is loaded on
 * that GPU and held until the process ends. The call allocates and frees nothing; its first
 * call on a device looks up that device's address of the array (hipGetSymbolAddress).
 *
 * Limit: gdn_prefill_segmented_workspace_bytes(dims, seg_t, 0) must not exceed
 * GDN_NOALLOC_SCRATCH_BYTES, else GDN_ERR_WORKSPACE and nothing is enqueued (at 32 V heads
 * of d = 128 segments of up to 1024 tokens fit). The array keeps whatever the last call on
 * the GPU left in it; every kernel that reads a workspace region writes it first within
 * the same call, so no call depends on its contents. All calls on one GPU share the one
 * array: two calls that overlap in time on the same GPU (different streams or host
 * threads with no ordering between them) race on it and give undefined results; calls on
 * one stream, or ordered by events, are safe. Other arguments and errors as for
 * gdn_prefill_segmented with overlapped = 0; GDN_ERR_HIP if the array's address cannot be
 * looked up.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (16u << 20)

size_t gdn_noalloc_scratch_bytes(void);
gdn_status gdn_prefill_segmented_noalloc(const gdn_dims* dims, int64_t seg_t, const void* q,
                                         const void* k, const void* v, const float* g,
                                         const float* beta, const float* state_in, float* out,
                                         float* state_out, void* stream);

/*
 * Calibration (measurement only): `blocks` workgroups of four waves each issue `iters`
 * rounds of four independent 32x32x16 bf16 MFMAs on `stream`, then write one float per
 * lane to `sink` (device memory of blocks x 256 floats, contents meaningless). The
 * achievable dense bf16 rate is gdn_calib_mfma_bf16_flops(iters, blocks) divided by the
 * launch time; the chunked kernels' MFMA rate is reported against it and against the
 * published peak. GDN_ERR_NULL for a NULL sink, GDN_ERR_SHAPE unless iters > 0 and
 * 0 < blocks <= 2^20, GDN_ERR_ALIGN for a sink not 4-byte aligned. The flop count is 0
 * for invalid arguments.
 */
int64_t gdn_calib_mfma_bf16_flops(int64_t iters, int32_t blocks);
gdn_status gdn_calib_mfma_bf16(int64_t iters, int32_t blocks, float* sink, void* stream);

/*
 * Calibration (measurement only): copy `bytes` (a positive multiple of 16) from src to dst,
 * both device pointers, 16-byte aligned and disjoint, with `blocks` workgroups of 256
 * threads sweeping the buffers in a grid-stride loop of 16-byte elements, on `stream`. The
 * achievable read + write rate of device memory is 2 * bytes divided by the launch time;
 * the decode step, which reads and writes each state element once, is reported against it
 * next to the published 8 TB/s. GDN_ERR_NULL, GDN_ERR_SHAPE (bytes or blocks out of range,
 * blocks at most 2^20), GDN_ERR_ALIGN, GDN_ERR_ALIAS (the ranges overlap).
 */
gdn_status gdn_calib_stream_copy(const void* src, void* dst, int64_t bytes, int32_t blocks,
                                 void* stream);

/*
 * Diagnostic (testing only): `blocks` workgroups, each holding the whole 160 KB of a CU's
 * LDS, fill it with the 32-bit `pattern` on `stream`. Launched with a few workgroups per
 * CU right before a kernel, it leaves that pattern wherever the kernel reads LDS it has not
 * written (with a NaN pattern, such a read shows up as a non-finite result). `sink` is
 * device memory of one uint32_t that the kernel writes only if the fill failed; its contents
 * are otherwise left as they are. GDN_ERR_NULL for a NULL sink, GDN_ERR_SHAPE unless
 * 0 < blocks <= 2^20, GDN_ERR_ALIGN for a sink not 4-byte aligned.
 */
gdn_status gdn_debug_fill_lds(uint32_t pattern, int32_t blocks, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
