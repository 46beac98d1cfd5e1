"""Python binding of libgdn.so: the Gated DeltaNet recurrence on MI355X (gfx950).

Thin ctypes wrappers with the same names as the C ABI in include/gdn.h. They check that
tensors are contiguous CUDA (HIP) tensors of the right dtype, allocate outputs and the
workspace with torch when the caller does not pass them, and hand raw device pointers and
the current stream to the library. Every step of the computation runs in the library's
HIP kernels; there is no Python or CPU fallback, and a missing libgdn.so is an error.

Layouts (see include/gdn.h): q, k [n, t, h_qk, d]; v [n, t, h_v, d]; g, beta [n, t, h_v]
fp32; state [n, h_v, d, d] fp32 with element [i][j] = S[j][i]; out [n, t, h_v, d] fp32.
"""
import ctypes
import os

import torch

__all__ = [
    "GdnError", "gdn_abi_version", "gdn_status_str", "gdn_workspace_bytes",
    "gdn_prefill_chunked", "gdn_prefill_scan", "gdn_decode_step", "gdn_prefill_choose",
    "gdn_prefill", "gdn_prefill_workspace_bytes", "library_path", "Dims", "BoundCall",
    "bind_prefill_chunked", "bind_prefill_scan", "bind_decode_step", "DecodeGraph",
    "gdn_prefill_segmented", "gdn_prefill_segmented_workspace_bytes", "gdn_prefill_scan_blockwise",
    "calib_mfma_bf16", "calib_stream_copy", "gdn_prefill_segmented_noalloc", "gdn_noalloc_scratch_bytes",
    "debug_fill_lds",
]

GDN_F32, GDN_BF16 = 0, 1
_DTYPES = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")
_lib = None


class Dims(ctypes.Structure):
    """gdn_dims from include/gdn.h."""
    _fields_ = [("n", ctypes.c_int64), ("t", ctypes.c_int64), ("h_qk", ctypes.c_int32),
                ("h_v", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("qkv_dtype", ctypes.c_int32), ("l2_eps", ctypes.c_float)]


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gdn_status_str(status)}")


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                           "(the HIP library is required, there is no fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, D = ctypes.c_void_p, ctypes.POINTER(Dims)
    i32, sz = ctypes.c_int32, ctypes.c_size_t
    sig = {
        "gdn_abi_version": (i32, []),
        "gdn_status_str": (ctypes.c_char_p, [ctypes.c_int32]),
        "gdn_workspace_bytes": (sz, [D, i32]),
        "gdn_prefill_chunked": (ctypes.c_int, [D, i32] + [P] * 9 + [sz, P]),
        "gdn_prefill_scan": (ctypes.c_int, [D] + [P] * 9 + [sz, P]),
        "gdn_decode_step": (ctypes.c_int, [D] + [P] * 9),
        "gdn_prefill_choose": (ctypes.c_int, [D, ctypes.POINTER(i32)]),
        "gdn_prefill_workspace_bytes": (sz, [D]),
        "gdn_prefill": (ctypes.c_int, [D] + [P] * 9 + [sz, P]),
        "gdn_decode_graph_create": (ctypes.c_int, [D, i32] + [ctypes.POINTER(P)] * 7 + [P, ctypes.POINTER(P)]),
        "gdn_graph_launch": (ctypes.c_int, [P, P]),
        "gdn_graph_destroy": (ctypes.c_int, [P]),
        "gdn_calib_mfma_bf16_flops": (ctypes.c_int64, [ctypes.c_int64, ctypes.c_int32]),
        "gdn_calib_mfma_bf16": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, P, P]),
        "gdn_prefill_scan_blockwise": (ctypes.c_int, [D, ctypes.c_int64] + [P] * 9 + [sz, P]),
        "gdn_prefill_segmented_workspace_bytes": (sz, [D, ctypes.c_int64, ctypes.c_int32]),
        "gdn_prefill_segmented": (ctypes.c_int, [D, ctypes.c_int64, ctypes.c_int32] + [P] * 9
                                  + [sz, P]),
        "gdn_noalloc_scratch_bytes": (sz, []),
        "gdn_calib_stream_copy": (ctypes.c_int, [P, P, ctypes.c_int64, ctypes.c_int32, P]),
        "gdn_prefill_segmented_noalloc": (ctypes.c_int, [D, ctypes.c_int64] + [P] * 9),
        "gdn_debug_fill_lds": (ctypes.c_int, [ctypes.c_uint32, ctypes.c_int32, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _lib = lib
    return lib


def gdn_abi_version() -> int:
    return _load().gdn_abi_version()


def gdn_status_str(status: int) -> str:
    return _load().gdn_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != 0:
        raise GdnError(status, where)


def make_dims(n, t, h_qk, h_v, d, dtype=torch.bfloat16, l2_eps=1e-6) -> Dims:
    return Dims(int(n), int(t), int(h_qk), int(h_v), int(d), int(d),
                _DTYPES.get(dtype, -1), float(l2_eps))


def _dims_of(q, v, l2_eps) -> Dims:
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [n, t, h_qk, d] and v [n, t, h_v, d]")
    n, t, h_qk, d_k = q.shape
    d = Dims(n, t, h_qk, v.shape[2], d_k, v.shape[3], _DTYPES.get(q.dtype, -1), float(l2_eps))
    return d


def _ptr(x):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _check_tensor(name, x, shape, dtype, dev):
    """x must be a contiguous CUDA (HIP) tensor on dev with exactly this shape and dtype."""
    if not isinstance(x, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if not x.is_cuda or x.device != dev:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor on {dev}")
    if x.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {x.dtype}")
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(x.shape)}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _prepare(q, k, v, g, beta, state_in, out, state_out, l2_eps):
    """Check every tensor of a call against the sizes q and v define (all before any
    launch: a wrong shape, dtype, device or layout would otherwise reach the kernels as a
    raw pointer) and allocate out / state_out when they are not given."""
    if not isinstance(q, torch.Tensor) or not isinstance(v, torch.Tensor):
        raise ValueError("q and v must be torch tensors")
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [n, t, h_qk, d] and v [n, t, h_v, d]")
    if q.dtype not in _DTYPES:
        raise ValueError("q, k, v must share one dtype, bfloat16 or float32")
    dev = q.device
    n, t, h_qk, d = q.shape
    h_v = v.shape[2]
    f32 = torch.float32
    _check_tensor("q", q, (n, t, h_qk, d), q.dtype, dev)
    _check_tensor("k", k, (n, t, h_qk, d), q.dtype, dev)
    _check_tensor("v", v, (n, t, h_v, v.shape[3]), q.dtype, dev)
    if v.shape[3] != d:
        raise ValueError(f"v must have shape {(n, t, h_v, d)}, got {tuple(v.shape)}")
    _check_tensor("g", g, (n, t, h_v), f32, dev)
    _check_tensor("beta", beta, (n, t, h_v), f32, dev)
    if state_in is not None:
        _check_tensor("state_in", state_in, (n, h_v, d, d), f32, dev)
    dims = _dims_of(q, v, l2_eps)
    if out is None:
        out = torch.empty((n, t, h_v, d), device=dev, dtype=f32)
    else:
        _check_tensor("out", out, (n, t, h_v, d), f32, dev)
    if state_out is None:
        state_out = torch.empty((n, h_v, d, d), device=dev, dtype=f32)
    else:
        _check_tensor("state_out", state_out, (n, h_v, d, d), f32, dev)
    return dims, out, state_out


def _check_workspace(workspace, dev):
    """A caller-supplied workspace: a contiguous uint8 tensor on the call's device."""
    if workspace is None:
        return 0
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8:
        raise ValueError("workspace must be a uint8 torch tensor")
    if not workspace.is_cuda or workspace.device != dev:
        raise ValueError(f"workspace must be a CUDA (HIP) tensor on {dev}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace.numel()


def _workspace(dims, chunk, workspace, dev):
    need = _load().gdn_workspace_bytes(ctypes.byref(dims), int(chunk))
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    return workspace, _check_workspace(workspace, dev)


def gdn_workspace_bytes(n, t, h_qk, h_v, d, dtype=torch.bfloat16, chunk=64) -> int:
    """Workspace bytes for gdn_prefill_chunked (chunk > 0) or gdn_prefill_scan (chunk 0)."""
    return _load().gdn_workspace_bytes(ctypes.byref(make_dims(n, t, h_qk, h_v, d, dtype)),
                                       int(chunk))


def gdn_prefill_chunked(q, k, v, g, beta, state_in=None, *, chunk=64, l2_eps=1e-6, out=None,
                        state_out=None, workspace=None, stream=None):
    """Chunked prefill. Returns (out, state_out)."""
    dims, out, state_out = _prepare(q, k, v, g, beta, state_in, out, state_out, l2_eps)
    workspace, wbytes = _workspace(dims, chunk, workspace, q.device)
    _check(_load().gdn_prefill_chunked(
        ctypes.byref(dims), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(workspace), wbytes,
        _stream(q.device, stream)), "gdn_prefill_chunked")
    return out, state_out


def gdn_prefill_scan(q, k, v, g, beta, state_in=None, *, l2_eps=1e-6, out=None,
                     state_out=None, workspace=None, stream=None):
    """Direct-scan prefill. Returns (out, state_out)."""
    dims, out, state_out = _prepare(q, k, v, g, beta, state_in, out, state_out, l2_eps)
    workspace, wbytes = _workspace(dims, 0, workspace, q.device)
    _check(_load().gdn_prefill_scan(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
        _ptr(out), _ptr(state_out), _ptr(workspace), wbytes, _stream(q.device, stream)),
        "gdn_prefill_scan")
    return out, state_out


def gdn_prefill_scan_blockwise(q, k, v, g, beta, state_in=None, *, block_t, l2_eps=1e-6,
                               out=None, state_out=None, workspace=None, stream=None):
    """The residency ablation of gdn_prefill_scan: one scan launch per block of block_t
    tokens, the state written to and read back from state_out between blocks. Returns
    (out, state_out)."""
    dims, out, state_out = _prepare(q, k, v, g, beta, state_in, out, state_out, l2_eps)
    workspace, wbytes = _workspace(dims, 0, workspace, q.device)
    _check(_load().gdn_prefill_scan_blockwise(
        ctypes.byref(dims), int(block_t), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(workspace), wbytes,
        _stream(q.device, stream)), "gdn_prefill_scan_blockwise")
    return out, state_out


def calib_mfma_bf16(iters, blocks, sink, stream=None) -> int:
    """Launch the bf16 MFMA loop (measurement only) into `sink` (a float32 device tensor of
    at least blocks * 256 elements); returns the flops the launch performs."""
    assert sink.dtype == torch.float32 and sink.is_cuda and sink.numel() >= blocks * 256
    _check(_load().gdn_calib_mfma_bf16(int(iters), int(blocks), _ptr(sink),
                                       _stream(sink.device, stream)), "gdn_calib_mfma_bf16")
    return int(_load().gdn_calib_mfma_bf16_flops(int(iters), int(blocks)))


def calib_stream_copy(src, dst, blocks=1024, stream=None):
    """Launch the streaming-copy calibration kernel (measurement only): dst <- src, two
    contiguous device tensors of the same byte size (a multiple of 16)."""
    nbytes = src.numel() * src.element_size()
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()
            and dst.numel() * dst.element_size() == nbytes):
        raise ValueError("src and dst must be contiguous device tensors of the same byte size")
    _check(_load().gdn_calib_stream_copy(_ptr(src), _ptr(dst), nbytes, int(blocks),
                                         _stream(src.device, stream)), "gdn_calib_stream_copy")


def debug_fill_lds(sink, pattern=0x7FC00000, blocks=1024, stream=None):
    """Fill the LDS of every CU with a 32-bit pattern (testing only; default a quiet NaN),
    so that a kernel launched next on the same stream that reads LDS it never wrote sees
    that pattern. `sink`: an int32 device tensor of at least one element, written only if
    the fill failed."""
    _check_tensor("sink", sink, (sink.numel(),), torch.int32, sink.device)
    if sink.numel() < 1:
        raise ValueError("sink: need at least one element")
    _check(_load().gdn_debug_fill_lds(int(pattern) & 0xFFFFFFFF, int(blocks), _ptr(sink),
                                      _stream(sink.device, stream)), "gdn_debug_fill_lds")


def gdn_decode_step(q, k, v, g, beta, state_in=None, *, l2_eps=1e-6, out=None,
                    state_out=None, stream=None):
    """One decode token per sequence (t == 1). Returns (out, state_out); pass
    state_out=state_in to update the state in place."""
    dims, out, state_out = _prepare(q, k, v, g, beta, state_in, out, state_out, l2_eps)
    _check(_load().gdn_decode_step(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
        _ptr(out), _ptr(state_out), _stream(q.device, stream)), "gdn_decode_step")
    return out, state_out


def gdn_prefill_choose(t, h_qk=16, h_v=32, d=128, n=1, dtype=torch.bfloat16) -> int:
    """The measured scan/chunk choice: 0 for the direct scan, else a chunk size."""
    res = ctypes.c_int32(-1)
    _check(_load().gdn_prefill_choose(ctypes.byref(make_dims(n, t, h_qk, h_v, d, dtype)),
                                      ctypes.byref(res)), "gdn_prefill_choose")
    return res.value


def gdn_prefill_workspace_bytes(n, t, h_qk, h_v, d, dtype=torch.bfloat16) -> int:
    return _load().gdn_prefill_workspace_bytes(ctypes.byref(make_dims(n, t, h_qk, h_v, d, dtype)))


def gdn_prefill(q, k, v, g, beta, state_in=None, *, l2_eps=1e-6, out=None, state_out=None,
                workspace=None, stream=None):
    """Prefill with the method gdn_prefill_choose picks. Returns (out, state_out)."""
    dims, out, state_out = _prepare(q, k, v, g, beta, state_in, out, state_out, l2_eps)
    if workspace is None:
        need = _load().gdn_prefill_workspace_bytes(ctypes.byref(dims))
        if need > 0:
            workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    wbytes = _check_workspace(workspace, q.device)
    _check(_load().gdn_prefill(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
        _ptr(out), _ptr(state_out), _ptr(workspace), wbytes, _stream(q.device, stream)),
        "gdn_prefill")
    return out, state_out


class BoundCall:
    """One library call with its arguments marshalled once (for loops that replay the same
    call, such as benchmarks or a layer stack). Calling it enqueues the kernels on the
    stream that was current at bind time and raises GdnError on a non-OK status."""

    def __init__(self, fn, args, where, keep):
        self._fn, self._args, self._where, self._keep = fn, args, where, keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise GdnError(st, self._where)


def bind_prefill_chunked(q, k, v, g, beta, state_in, out, state_out, workspace, *, chunk=64,
                         l2_eps=1e-6, stream=None) -> BoundCall:
    dims, out, state_out = _prepare(q, k, v, g, beta, state_in, out, state_out, l2_eps)
    nbytes = _check_workspace(workspace, q.device)
    args = (ctypes.byref(dims), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(workspace), nbytes,
            _stream(q.device, stream))
    return BoundCall(_load().gdn_prefill_chunked, args, "gdn_prefill_chunked",
                     (dims, q, k, v, g, beta, state_in, out, state_out, workspace))


def bind_prefill_scan(q, k, v, g, beta, state_in, out, state_out, workspace, *, l2_eps=1e-6,
                      stream=None) -> BoundCall:
    dims, out, state_out = _prepare(q, k, v, g, beta, state_in, out, state_out, l2_eps)
    nbytes = _check_workspace(workspace, q.device)
    args = (ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
            _ptr(out), _ptr(state_out), _ptr(workspace), nbytes, _stream(q.device, stream))
    return BoundCall(_load().gdn_prefill_scan, args, "gdn_prefill_scan",
                     (dims, q, k, v, g, beta, state_in, out, state_out, workspace))


def bind_decode_step(q, k, v, g, beta, state_in, out, state_out, *, l2_eps=1e-6,
                     stream=None) -> BoundCall:
    dims, out, state_out = _prepare(q, k, v, g, beta, state_in, out, state_out, l2_eps)
    args = (ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
            _ptr(out), _ptr(state_out), _stream(q.device, stream))
    return BoundCall(_load().gdn_decode_step, args, "gdn_decode_step",
                     (dims, q, k, v, g, beta, state_in, out, state_out))


def gdn_prefill_segmented_workspace_bytes(n, t, h_qk, h_v, d, seg_t, overlapped=False,
                                          dtype=torch.bfloat16) -> int:
    return _load().gdn_prefill_segmented_workspace_bytes(
        ctypes.byref(make_dims(n, t, h_qk, h_v, d, dtype)), int(seg_t), int(bool(overlapped)))


def gdn_prefill_segmented(q, k, v, g, beta, state_in=None, *, seg_t, overlapped=False,
                          l2_eps=1e-6, out=None, state_out=None, workspace=None, stream=None):
    """Prefill as consecutive segments of seg_t tokens per sequence with one reused
    workspace (sized by seg_t; two segment slots when overlapped, so that a segment's
    per-chunk preparation runs on a side stream during the previous segment's sequential
    pass). Returns (out, state_out)."""
    dims, out, state_out = _prepare(q, k, v, g, beta, state_in, out, state_out, l2_eps)
    ov = int(bool(overlapped))
    if workspace is None:
        need = _load().gdn_prefill_segmented_workspace_bytes(ctypes.byref(dims), int(seg_t), ov)
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    wbytes = _check_workspace(workspace, q.device)
    _check(_load().gdn_prefill_segmented(
        ctypes.byref(dims), int(seg_t), ov, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(workspace), wbytes,
        _stream(q.device, stream)), "gdn_prefill_segmented")
    return out, state_out


def gdn_noalloc_scratch_bytes() -> int:
    """Size of the library's static per-GPU workspace used by gdn_prefill_segmented_noalloc."""
    return int(_load().gdn_noalloc_scratch_bytes())


def gdn_prefill_segmented_noalloc(q, k, v, g, beta, state_in=None, *, seg_t, l2_eps=1e-6,
                                  out, state_out, stream=None):
    """gdn_prefill_segmented (in order) with the library's static workspace instead of a
    caller's: the library allocates nothing. The caller passes the outputs. Returns
    (out, state_out)."""
    dims, out, state_out = _prepare(q, k, v, g, beta, state_in, out, state_out, l2_eps)
    _check(_load().gdn_prefill_segmented_noalloc(
        ctypes.byref(dims), int(seg_t), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(state_in), _ptr(out), _ptr(state_out), _stream(q.device, stream)),
        "gdn_prefill_segmented_noalloc")
    return out, state_out


class DecodeGraph:
    """gdn_decode_graph_create / gdn_graph_launch / gdn_graph_destroy: one decode token
    through len(q) stacked layers as dependent per-layer steps, recorded once as a HIP
    graph. Each layer's inputs are [n, 1, ...] tensors as for gdn_decode_step; its state
    (state[i]) is updated in place and its output written to out[i] (allocated when not
    given). The tensors are referenced by address: write each token's inputs into them in
    place and call launch(). `stream` (a non-default torch stream) is used only to record.
    """

    def __init__(self, q, k, v, g, beta, state, out=None, *, l2_eps=1e-6, stream):
        layers = len(q)
        if not all(len(x) == layers for x in (k, v, g, beta, state)):
            raise ValueError("one tensor per layer in every list")
        if out is None:
            out = [torch.empty(v[i].shape, device=v[i].device, dtype=torch.float32)
                   for i in range(layers)]
        for i in range(layers):
            _prepare(q[i], k[i], v[i], g[i], beta[i], state[i], out[i], state[i], l2_eps)
            # one gdn_dims describes every layer: each layer must match layer 0 exactly
            if (q[i].shape != q[0].shape or v[i].shape != v[0].shape
                    or q[i].dtype != q[0].dtype or q[i].device != q[0].device):
                raise ValueError(f"layer {i}: q/v shapes, dtype and device must equal layer 0's")
        self.tensors = (list(q), list(k), list(v), list(g), list(beta), list(state), list(out))
        self.out = self.tensors[6]
        dims = _dims_of(q[0], v[0], l2_eps) if layers else make_dims(0, 1, 1, 1, 16)
        arr = lambda xs: (ctypes.c_void_p * max(1, layers))(*[x.data_ptr() for x in xs])
        self._arrays = [arr(xs) for xs in self.tensors]
        handle = ctypes.c_void_p()
        _check(_load().gdn_decode_graph_create(
            ctypes.byref(dims), layers, *[ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p)) for a in self._arrays],
            ctypes.c_void_p(stream.cuda_stream), ctypes.byref(handle)), "gdn_decode_graph_create")
        self._handle = handle

    def launch(self, stream=None):
        dev = self.tensors[0][0].device if self.tensors[0] else None
        _check(_load().gdn_graph_launch(self._handle, _stream(dev, stream)), "gdn_graph_launch")

    def close(self):
        if getattr(self, "_handle", None) is not None and self._handle.value:
            _check(_load().gdn_graph_destroy(self._handle), "gdn_graph_destroy")
        self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
