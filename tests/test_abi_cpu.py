"""CPU tests of the C ABI: the library loads, exports every symbol include/gdn.h declares,
and every validation path returns its error code before any HIP call (no GPU needed).

Pointers below are fake device addresses: validation never dereferences them, and every
call here fails validation, so nothing is launched.
"""
import ctypes
import os
import re
import subprocess

import pytest

import gated_deltanet_linear_prefill_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, WS, HIP = range(8)
MB = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return gdn._load()


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"gdn_prefill_chunked", "gdn_prefill_scan", "gdn_decode_step",
            "gdn_prefill_choose", "gdn_workspace_bytes", "gdn_status_str"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    dyn = subprocess.run(["nm", "-D", "--defined-only", gdn.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gdn_\w+)", dyn))
    assert set(names) <= exported, set(names) - exported


def test_abi_version(lib):
    m = re.search(r"#define GDN_ABI_VERSION (\d+)", open(HEADER).read())
    assert gdn.gdn_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for code in range(8):
        s = gdn.gdn_status_str(code)
        assert s.startswith("GDN_") and len(s) > 10
    assert "unknown" in gdn.gdn_status_str(99)


class Bufs:
    """Disjoint, 256-byte aligned fake device ranges for one call."""

    def __init__(self, n=1, t=64, h_qk=2, h_v=4, d=32, esize=2):
        base = 0x7F0000000000
        sizes = dict(q=n * t * h_qk * d * esize, k=n * t * h_qk * d * esize,
                     v=n * t * h_v * d * esize, g=n * t * h_v * 4, beta=n * t * h_v * 4,
                     state_in=n * h_v * d * d * 4, out=n * t * h_v * d * 4,
                     state_out=n * h_v * d * d * 4, ws=64 * MB)
        self.addr = {}
        for key, size in sizes.items():
            self.addr[key] = base
            base += (size + 4095) // 4096 * 4096 + 4096
        self.dims = gdn.make_dims(n, t, h_qk, h_v, d, gdn.torch.bfloat16 if esize == 2
                                  else gdn.torch.float32)

    def p(self, key, off=0):
        return ctypes.c_void_p(self.addr[key] + off)


def call_chunked(lib, b, chunk=64, dims=None, ws_bytes=64 * MB, **over):
    a = {key: b.p(key) for key in ("q", "k", "v", "g", "beta", "state_in", "out",
                                    "state_out", "ws")}
    a.update(over)
    d = ctypes.byref(dims if dims is not None else b.dims)
    return lib.gdn_prefill_chunked(d, chunk, a["q"], a["k"], a["v"], a["g"], a["beta"],
                                   a["state_in"], a["out"], a["state_out"], a["ws"],
                                   ws_bytes, None)


def call_scan(lib, b, dims=None, ws_bytes=64 * MB, **over):
    a = {key: b.p(key) for key in ("q", "k", "v", "g", "beta", "state_in", "out",
                                    "state_out", "ws")}
    a.update(over)
    d = ctypes.byref(dims if dims is not None else b.dims)
    return lib.gdn_prefill_scan(d, a["q"], a["k"], a["v"], a["g"], a["beta"], a["state_in"],
                                a["out"], a["state_out"], a["ws"], ws_bytes, None)


def call_decode(lib, b, dims=None, **over):
    a = {key: b.p(key) for key in ("q", "k", "v", "g", "beta", "state_in", "out", "state_out")}
    a.update(over)
    d = ctypes.byref(dims if dims is not None else b.dims)
    return lib.gdn_decode_step(d, a["q"], a["k"], a["v"], a["g"], a["beta"], a["state_in"],
                               a["out"], a["state_out"], None)


def with_dims(b, **kw):
    d = gdn.Dims.from_buffer_copy(b.dims)
    for key, val in kw.items():
        setattr(d, key, val)
    return d


CALLS = [call_chunked, call_scan]


@pytest.mark.parametrize("call", CALLS + [call_decode], ids=["chunked", "scan", "decode"])
def test_null_dims(lib, call):
    b = Bufs(t=1)
    if call is call_decode:
        st = lib.gdn_decode_step(None, *[b.p("q")] * 8, None)
    elif call is call_scan:
        st = lib.gdn_prefill_scan(None, *[b.p("q")] * 9, 0, None)
    else:
        st = lib.gdn_prefill_chunked(None, 64, *[b.p("q")] * 9, 0, None)
    assert st == NULL


@pytest.mark.parametrize("call", CALLS, ids=["chunked", "scan"])
@pytest.mark.parametrize("field,value,code", [
    ("n", -1, SHAPE), ("t", -5, SHAPE), ("h_qk", 0, SHAPE), ("h_v", 3, SHAPE),
    ("h_v", -4, SHAPE), ("d_k", 48, UNSUP), ("d_v", 64, UNSUP), ("qkv_dtype", 7, UNSUP),
    ("l2_eps", -1.0, SHAPE), ("l2_eps", float("nan"), SHAPE), ("t", 1 << 62, SHAPE),
])
def test_bad_dims(lib, call, field, value, code):
    b = Bufs()
    kw = {field: value}
    if field == "d_k":
        kw["d_v"] = value
    assert call(lib, b, dims=with_dims(b, **kw)) == code


def test_bad_chunk(lib):
    b = Bufs()
    for chunk in (0, 8, 48, 256, -64):
        assert call_chunked(lib, b, chunk=chunk) == UNSUP


def test_decode_needs_one_token(lib):
    b = Bufs(t=2)
    assert call_decode(lib, b) == SHAPE
    b = Bufs(t=1)
    assert call_decode(lib, b, dims=with_dims(b, t=0)) == SHAPE


@pytest.mark.parametrize("call", CALLS + [call_decode], ids=["chunked", "scan", "decode"])
@pytest.mark.parametrize("key", ["q", "k", "v", "g", "beta", "out", "state_out"])
def test_missing_pointer(lib, call, key):
    b = Bufs(t=1)
    assert call(lib, b, **{key: None}) == NULL


@pytest.mark.parametrize("call", CALLS + [call_decode], ids=["chunked", "scan", "decode"])
@pytest.mark.parametrize("key,off", [("q", 2), ("k", 8), ("v", 4), ("state_in", 4),
                                     ("out", 8), ("state_out", 12), ("g", 2), ("beta", 1)])
def test_misaligned_pointer(lib, call, key, off):
    b = Bufs(t=1)
    assert call(lib, b, **{key: b.p(key, off)}) == ALIGN


def test_misaligned_workspace(lib):
    b = Bufs()
    assert call_chunked(lib, b, ws=b.p("ws", 8)) == ALIGN
    assert call_scan(lib, b, ws=b.p("ws", 4)) == ALIGN


def test_workspace_checks(lib):
    b = Bufs()
    need = lib.gdn_workspace_bytes(ctypes.byref(b.dims), 64)
    assert need > 0
    assert call_chunked(lib, b, ws=None) == WS
    assert call_chunked(lib, b, ws_bytes=need - 1) == WS


def test_scan_needs_no_workspace(lib):
    """The direct scan stages and normalises its inputs in LDS: no workspace at any size."""
    for t in (1, 2, 100, 4096, 131072):
        dims = gdn.make_dims(2, t, 16, 32, 128)
        assert lib.gdn_workspace_bytes(ctypes.byref(dims), 0) == 0


@pytest.mark.parametrize("call", CALLS + [call_decode], ids=["chunked", "scan", "decode"])
def test_aliasing(lib, call):
    b = Bufs(t=1)
    # out overlapping an input, the state, or state_out
    assert call(lib, b, out=b.p("v")) == ALIAS
    assert call(lib, b, out=b.p("q", 16)) == ALIAS
    assert call(lib, b, out=b.p("state_out")) == ALIAS
    assert call(lib, b, state_out=b.p("g")) == ALIAS
    # state_out partly overlapping state_in (equality is allowed; a shift is not)
    assert call(lib, b, state_out=b.p("state_in", 16)) == ALIAS
    assert call(lib, b, out=b.p("state_in")) == ALIAS


def test_workspace_alias(lib):
    """A workspace that overlaps any buffer of the call (the direct scan takes none, so
    its workspace arguments are not checked)."""
    b = Bufs()
    assert call_chunked(lib, b, ws=b.p("out")) == ALIAS
    assert call_chunked(lib, b, ws=b.p("state_in")) == ALIAS
    assert call_chunked(lib, b, ws=b.p("k")) == ALIAS


def test_zero_sequences_is_a_noop(lib):
    b = Bufs()
    # n == 0 with no buffers at all: nothing to do, nothing launched.
    z = with_dims(b, n=0)
    none = {key: None for key in ("q", "k", "v", "g", "beta", "state_in", "out",
                                   "state_out", "ws")}
    assert call_chunked(lib, b, dims=z, ws_bytes=0, **none) == OK
    assert call_scan(lib, b, dims=z, ws_bytes=0, **none) == OK
    assert call_decode(lib, b, dims=with_dims(b, n=0, t=1),
                       **{key: None for key in none if key != "ws"}) == OK


def test_workspace_bytes_queries(lib):
    b = Bufs(t=4096, h_qk=16, h_v=32, d=128)
    for chunk in (0, 16, 32, 64, 128):
        assert lib.gdn_workspace_bytes(ctypes.byref(b.dims), chunk) >= 0
    assert lib.gdn_workspace_bytes(ctypes.byref(b.dims), 48) == 0
    assert lib.gdn_workspace_bytes(None, 64) == 0
    assert lib.gdn_workspace_bytes(ctypes.byref(with_dims(b, d_k=40, d_v=40)), 64) == 0
    assert lib.gdn_workspace_bytes(ctypes.byref(with_dims(b, t=0)), 64) == 0


def test_prefill_choose(lib):
    for t in (1, 7, 64, 256, 4096, 131072):
        c = gdn.gdn_prefill_choose(t)
        assert c in (0, 16, 32, 64, 128)
    # The pick follows the measured table (the last entry whose min_t <= t), at and around
    # every boundary the table lists.
    inc = open(os.path.join(ROOT, "gated_deltanet_linear_prefill_amd", "csrc", "gdn_crossover.inc")).read()
    table = [(int(a), int(b)) for a, b in re.findall(r"\{(\d+), (\d+)\}", inc)]
    assert table and table[0][0] == 0 and [m for m, _ in table] == sorted(m for m, _ in table)

    def pick(t):
        return [ch for m, ch in table if m <= t][-1]

    for t in sorted({1, 2, 131072} | {m + dt for m, _ in table for dt in (-1, 0, 1) if m + dt >= 1}):
        assert gdn.gdn_prefill_choose(t) == pick(t), t
    res = ctypes.c_int32()
    assert lib.gdn_prefill_choose(None, ctypes.byref(res)) == NULL
    b = Bufs()
    assert lib.gdn_prefill_choose(ctypes.byref(b.dims), None) == NULL
    assert lib.gdn_prefill_choose(ctypes.byref(with_dims(b, h_v=3)), ctypes.byref(res)) == SHAPE


def test_python_wrappers_reject_cpu_tensors():
    import gdn_inputs
    c = gdn_inputs.make_case(gdn_inputs.TINY, seed=1)
    with pytest.raises(ValueError):
        gdn.gdn_prefill_scan(c["q"], c["k"], c["v"], c["g"], c["beta"])


# ------------------------------------------------------------------ decode graph (no GPU)
def graph_args(layers, bufs, **over):
    """Host arrays of per-layer fake device pointers for gdn_decode_graph_create."""
    keys = ("q", "k", "v", "g", "beta", "state_in", "out")
    arrays = []
    for key in keys:
        vals = [bufs[i].addr[key] for i in range(layers)]
        if key in over:
            vals = over[key](vals)
        arrays.append((ctypes.c_void_p * max(1, layers))(*vals))
    return [ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p)) for a in arrays]


def create_graph(lib, layers, bufs, dims, stream=ctypes.c_void_p(0x1000), handle=None, **over):
    h = handle if handle is not None else ctypes.c_void_p(0xDEAD)
    st = lib.gdn_decode_graph_create(ctypes.byref(dims), layers, *graph_args(layers, bufs, **over),
                                     stream, ctypes.byref(h))
    return st, h


def test_decode_graph_validation(lib):
    """Every layer is validated before anything is recorded (so no HIP call happens here);
    the handle is cleared on error."""
    bufs = [Bufs(t=1) for _ in range(3)]
    dims = bufs[0].dims
    st, h = create_graph(lib, 3, bufs, dims, stream=None)
    assert st == NULL and not h.value                           # no stream to record on
    st, h = create_graph(lib, 3, bufs, with_dims(bufs[0], t=2))
    assert st == SHAPE and not h.value                          # decode is one token
    st, h = create_graph(lib, 3, bufs, dims, q=lambda xs: xs[:2] + [None])
    assert st == NULL and not h.value                           # layer 2 has no q
    st, h = create_graph(lib, 3, bufs, dims, out=lambda xs: [xs[0], xs[1] + 4, xs[2]])
    assert st == ALIGN and not h.value                          # layer 1 misaligned out
    st, h = create_graph(lib, 3, bufs, dims, out=lambda xs: [xs[0], xs[1], bufs[2].addr["state_in"]])
    assert st == ALIAS and not h.value                          # layer 2 out overlaps its state
    st, h = create_graph(lib, -1, bufs, dims)
    assert st == SHAPE and not h.value
    assert lib.gdn_decode_graph_create(ctypes.byref(dims), 1, *graph_args(1, bufs),
                                       ctypes.c_void_p(0x1000), None) == NULL
    assert lib.gdn_graph_launch(None, None) == NULL
    assert lib.gdn_graph_destroy(None) == OK


# ------------------------------------------------------------------ segmented prefill (no GPU)
def call_segmented(lib, b, seg_t=16, dims=None, ws_bytes=64 * MB, overlapped=0, **over):
    a = {key: b.p(key) for key in ("q", "k", "v", "g", "beta", "state_in", "out",
                                    "state_out", "ws")}
    a.update(over)
    d = ctypes.byref(dims if dims is not None else b.dims)
    return lib.gdn_prefill_segmented(d, seg_t, overlapped, a["q"], a["k"], a["v"], a["g"], a["beta"],
                                     a["state_in"], a["out"], a["state_out"], a["ws"],
                                     ws_bytes, None)


def test_segmented_validation(lib):
    """The whole call is validated before any segment is issued (no HIP call here)."""
    b = Bufs(t=256)
    seg = 64  # segments dispatched to the chunked path, which needs a workspace
    assert gdn.gdn_prefill_choose(seg, b.dims.h_qk, b.dims.h_v, b.dims.d_k, 1) > 0
    assert lib.gdn_prefill_segmented(None, 16, 0, *[None] * 9, 0, None) == NULL
    assert call_segmented(lib, b, seg_t=0) == SHAPE
    assert call_segmented(lib, b, seg_t=-5) == SHAPE
    assert call_segmented(lib, b, seg_t=seg, overlapped=2) == SHAPE
    assert call_segmented(lib, b, seg_t=seg, overlapped=-1) == SHAPE
    need = lib.gdn_prefill_segmented_workspace_bytes(ctypes.byref(b.dims), seg, 1)
    assert call_segmented(lib, b, seg_t=seg, overlapped=1, ws_bytes=need - 1) == WS
    assert call_segmented(lib, b, seg_t=seg, overlapped=1, ws=b.p("ws", 8)) == ALIGN
    assert call_segmented(lib, b, seg_t=seg, q=None) == NULL
    assert call_segmented(lib, b, seg_t=seg, out=b.p("out", 4)) == ALIGN
    assert call_segmented(lib, b, seg_t=seg, out=b.p("q")) == ALIAS
    assert call_segmented(lib, b, seg_t=seg, ws=None) == WS
    assert call_segmented(lib, b, seg_t=seg, ws_bytes=16) == WS
    assert call_segmented(lib, b, seg_t=seg, ws=b.p("state_out")) == ALIAS
    assert call_segmented(lib, b, seg_t=seg, dims=with_dims(b, d_k=40, d_v=40)) == UNSUP


def test_segmented_workspace_bytes(lib):
    """The segmented workspace depends on the segment length, not on t."""
    long = gdn.make_dims(2, 131072, 16, 32, 128)
    seg = lib.gdn_prefill_segmented_workspace_bytes(ctypes.byref(long), 4096, 0)
    one = lib.gdn_prefill_workspace_bytes(ctypes.byref(gdn.make_dims(1, 4096, 16, 32, 128)))
    assert seg == one > 0
    assert lib.gdn_prefill_segmented_workspace_bytes(ctypes.byref(long), 0, 0) == 0
    ragged = gdn.make_dims(1, 4096 + 100, 16, 32, 128)
    last = lib.gdn_prefill_workspace_bytes(ctypes.byref(gdn.make_dims(1, 100, 16, 32, 128)))
    assert lib.gdn_prefill_segmented_workspace_bytes(ctypes.byref(ragged), 4096, 0) == max(one, last)
    # overlapped: two slots, each rounded up to 256 bytes
    slot = (max(one, last) + 255) // 256 * 256
    assert lib.gdn_prefill_segmented_workspace_bytes(ctypes.byref(ragged), 4096, 1) == 2 * slot
    assert lib.gdn_prefill_segmented_workspace_bytes(ctypes.byref(ragged), 4096, 2) == 0


# ------------------------------------------------------------------ blockwise scan ablation (no GPU)
def test_scan_blockwise_validation(lib):
    """Validated like gdn_prefill_scan before any launch; block_t must be positive."""
    b = Bufs(t=64)
    a = {key: b.p(key) for key in ("q", "k", "v", "g", "beta", "state_in", "out", "state_out",
                                    "ws")}

    def call(block_t=16, ws_bytes=64 * MB, **over):
        x = dict(a, **over)
        return lib.gdn_prefill_scan_blockwise(ctypes.byref(b.dims), block_t, x["q"], x["k"],
                                              x["v"], x["g"], x["beta"], x["state_in"],
                                              x["out"], x["state_out"], x["ws"], ws_bytes, None)

    assert lib.gdn_prefill_scan_blockwise(None, 16, *[None] * 9, 0, None) == NULL
    assert call(block_t=0) == SHAPE
    assert call(block_t=-1) == SHAPE
    assert call(q=None) == NULL
    assert call(out=b.p("q")) == ALIAS
    assert call(out=b.p("out", 4)) == ALIGN


# ------------------------------------------------------------------ MFMA calibration loop (no GPU)
def test_calib_validation(lib):
    """Arguments are checked before any launch; the flop count follows the loop's shape."""
    sink = ctypes.c_void_p(0x100000)
    assert lib.gdn_calib_mfma_bf16(10, 4, None, None) == NULL
    assert lib.gdn_calib_mfma_bf16(0, 4, sink, None) == SHAPE
    assert lib.gdn_calib_mfma_bf16(10, 0, sink, None) == SHAPE
    assert lib.gdn_calib_mfma_bf16(10, (1 << 20) + 1, sink, None) == SHAPE
    assert lib.gdn_calib_mfma_bf16(10, 4, ctypes.c_void_p(0x100002), None) == ALIGN
    assert lib.gdn_calib_mfma_bf16_flops(10, 4) == 4 * 4 * 10 * 4 * 32 * 32 * 16 * 2
    assert lib.gdn_calib_mfma_bf16_flops(0, 4) == 0
    assert lib.gdn_calib_mfma_bf16_flops(10, -1) == 0


def test_single_token_prefill_needs_no_workspace(lib):
    """gdn_prefill runs one token as the decode step and short prompts as the direct scan,
    which need no workspace; the segmented workspace for one-token segments is therefore 0
    as well. Lengths dispatched to the chunked path need one."""
    one = gdn.make_dims(2, 1, 16, 32, 128)
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(one)) == 0
    two = gdn.make_dims(2, 2, 16, 32, 128)
    assert gdn.gdn_prefill_choose(2, 16, 32, 128, 2) == 0
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(two)) == 0
    long = gdn.make_dims(2, 4096, 16, 32, 128)
    assert gdn.gdn_prefill_choose(4096, 16, 32, 128, 2) > 0
    assert lib.gdn_prefill_workspace_bytes(ctypes.byref(long)) > 0
    seq = gdn.make_dims(1, 100, 16, 32, 128)
    assert lib.gdn_prefill_segmented_workspace_bytes(ctypes.byref(seq), 1, 0) == 0


# ------------------------------------------------------------- allocation-free entry (no GPU)
def call_noalloc(lib, b, seg_t=16, dims=None, **over):
    a = {key: b.p(key) for key in ("q", "k", "v", "g", "beta", "state_in", "out", "state_out")}
    a.update(over)
    d = ctypes.byref(dims if dims is not None else b.dims)
    return lib.gdn_prefill_segmented_noalloc(d, seg_t, a["q"], a["k"], a["v"], a["g"],
                                             a["beta"], a["state_in"], a["out"],
                                             a["state_out"], None)


def test_noalloc_validation(lib):
    """Every error of the allocation-free entry is returned before its scratch lookup or any
    launch (no HIP call here): the segmented checks, and a segment whose workspace exceeds
    the static array."""
    assert lib.gdn_noalloc_scratch_bytes() == 16 << 20
    b = Bufs(t=64)
    assert lib.gdn_prefill_segmented_noalloc(None, 16, *[None] * 8, None) == NULL
    assert call_noalloc(lib, b, seg_t=0) == SHAPE
    assert call_noalloc(lib, b, seg_t=-1) == SHAPE
    assert call_noalloc(lib, b, q=None) == NULL
    assert call_noalloc(lib, b, out=b.p("out", 4)) == ALIGN
    assert call_noalloc(lib, b, out=b.p("q")) == ALIAS
    assert call_noalloc(lib, b, state_out=b.p("out")) == ALIAS
    assert call_noalloc(lib, b, dims=with_dims(b, d_k=40, d_v=40)) == UNSUP
    # the 4K workload: 1024-token segments fit the 16 MiB array, 2048-token ones do not
    big = Bufs(t=4096, h_qk=16, h_v=32, d=128)
    fit = lib.gdn_prefill_segmented_workspace_bytes(ctypes.byref(big.dims), 1024, 0)
    over = lib.gdn_prefill_segmented_workspace_bytes(ctypes.byref(big.dims), 2048, 0)
    assert 0 < fit <= lib.gdn_noalloc_scratch_bytes() < over
    assert call_noalloc(lib, big, seg_t=2048) == WS
    assert call_noalloc(lib, big, seg_t=4096) == WS


def test_calib_stream_copy_validation(lib):
    """Argument checks of the streaming-copy calibration (no launch on any error)."""
    P = ctypes.c_void_p
    a, b = P(0x7F0000000000), P(0x7F0000100000)
    f = lib.gdn_calib_stream_copy
    assert f(None, b, 1024, 16, None) == NULL
    assert f(a, None, 1024, 16, None) == NULL
    assert f(a, b, 0, 16, None) == SHAPE
    assert f(a, b, 1000, 16, None) == SHAPE
    assert f(a, b, 1024, 0, None) == SHAPE
    assert f(a, b, 1024, (1 << 20) + 1, None) == SHAPE
    assert f(P(0x7F0000000008), b, 1024, 16, None) == ALIGN
    assert f(a, P(0x7F0000000200), 1024, 16, None) == ALIAS


def test_debug_fill_lds_validation(lib):
    """Argument checks of the LDS fill diagnostic (no launch on any error)."""
    P = ctypes.c_void_p
    f = lib.gdn_debug_fill_lds
    assert f(0x7FC00000, 16, None, None) == NULL
    assert f(0x7FC00000, 0, P(0x7F0000000000), None) == SHAPE
    assert f(0x7FC00000, (1 << 20) + 1, P(0x7F0000000000), None) == SHAPE
    assert f(0x7FC00000, 16, P(0x7F0000000002), None) == ALIGN
