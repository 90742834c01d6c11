"""Python binding of libq4stream (MI355X / gfx950 INT4 weight-streaming decode).

Argument marshalling only: every step runs in the HIP kernels of
``libq4stream.so``.  PyTorch supplies device memory, pinned host memory and
streams; tensors are passed by pointer, streams by their HIP handle.

The names mirror ``include/q4.h``.  Any non-OK status raises ``Q4Error``;
a missing library raises ``RuntimeError`` -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "Q4Error", "lib", "abi_version",
    "q4_pack", "q4_unpack", "q4_gemv", "q4_gemm_smallbatch", "q4_gemv_tuned",
    "q4_gemm_tuned", "q4_gemm_valu", "q4_gemv_rows_tuned", "q4_gemv_rowp_tuned", "Decoder", "WeightStream", "layer_blob_layout",
    "decode_step_graph", "weight_stream_begin", "weight_stream_wait",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4stream.so")

STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "HIP", 4: "STATE", 5: "OOM"}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


class Q4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Matrix(ctypes.Structure):
    _fields_ = [("packed", _P), ("scales", _P), ("N", _I64), ("K", _I64)]


class Layer(ctypes.Structure):
    _fields_ = [("qkv", Matrix), ("o", Matrix), ("gate_up", Matrix), ("down", Matrix)]


class ModelDesc(ctypes.Structure):
    _fields_ = [("n_layers", _I32), ("d_model", _I32), ("n_heads", _I32),
                ("n_kv_heads", _I32), ("head_dim", _I32), ("d_ff", _I32),
                ("eps", ctypes.c_float), ("layers", ctypes.POINTER(Layer)),
                ("h", _P), ("workspace", _P), ("workspace_bytes", ctypes.c_size_t),
                ("kv_cache", _P), ("max_ctx", _I32), ("rope_base", ctypes.c_float),
                ("max_batch", _I32), ("h_batch", _P)]


class WStreamDesc(ctypes.Structure):
    _fields_ = [("n_layers", _I32), ("host_blobs", ctypes.POINTER(_P)),
                ("blob_bytes", ctypes.POINTER(ctypes.c_size_t)), ("slot", _P * 2),
                ("slot_bytes", ctypes.c_size_t), ("copy", _P), ("copy2", _P),
                ("chunk_bytes", ctypes.c_size_t), ("resident", ctypes.POINTER(_P))]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libq4stream.so (built in-tree by ``build.py``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m "
            "int4_weight_streaming_q4_amd.build` (no fallback path exists)")
    L = ctypes.CDLL(LIB_PATH)
    S = _I32
    sigs = {
        "q4_last_error": (ctypes.c_char_p, []),
        "q4_abi_version": (_I32, []),
        "q4_pack": (S, [_P, _P, _I64, _I64, _P]),
        "q4_unpack": (S, [_P, _P, _I64, _I64, _P]),
        "q4_quantize": (S, [_P, _I32, _P, _P, _I64, _I64, _P]),
        "q4_gemv": (S, [_P, _P, _P, _P, _I64, _I64, _P]),
        "q4_gemm_smallbatch": (S, [_P, _P, _P, _P, _I64, _I64, _I32, _P]),
        "q4_gemv_tuned": (S, [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _P]),
        "q4_gemm_tuned": (S, [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _P]),
        "q4_gemm_valu": (S, [_P, _P, _P, _P, _I64, _I64, _I32, _P]),
        "q4_gemv_rows_tuned": (S, [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _P]),
        "q4_gemv_rowp_tuned": (S, [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _P]),
        "q4_decoder_workspace_bytes": (S, [ctypes.POINTER(ModelDesc),
                                           ctypes.POINTER(ctypes.c_size_t)]),
        "q4_decoder_create": (S, [ctypes.POINTER(ModelDesc), ctypes.POINTER(_P)]),
        "decode_step_graph": (S, [_P, _I32, _P]),
        "q4_decode_step_eager": (S, [_P, _P]),
        "q4_decode_step_profiled": (S, [_P, _P, ctypes.POINTER(ctypes.c_float), _I32,
                                        ctypes.POINTER(_I32)]),
        "q4_decode_layer": (S, [_P, ctypes.POINTER(Layer), _P]),
        "q4_decode_layer_part": (S, [_P, ctypes.POINTER(Layer), _I32, _P]),
        "q4_decode_kernel_time": (S, [_P, _I32, _I32, _P, ctypes.POINTER(ctypes.c_float)]),
        "q4_decoder_destroy": (S, [_P]),
        "q4_decoder_set_persistent": (S, [_P, _I32]),
        "q4_decoder_check": (S, [_P]),
        "q4_decoder_set_context": (S, [_P, _I32, _P]),
        "q4_decode_verify_eager": (S, [_P, _I32, _P]),
        "q4_decode_verify_graph": (S, [_P, _I32, _P]),
        "q4_layer_blob_layout": (S, [ctypes.POINTER(Layer), ctypes.c_size_t * 8,
                                     ctypes.POINTER(ctypes.c_size_t)]),
        "q4_layer_from_blob": (S, [ctypes.POINTER(Layer), _P, ctypes.POINTER(Layer)]),
        "q4_wstream_create": (S, [ctypes.POINTER(WStreamDesc), ctypes.POINTER(_P)]),
        "q4_offload_plan": (S, [_I32, ctypes.c_size_t, ctypes.c_size_t, ctypes.POINTER(_I32),
                                ctypes.POINTER(_I32)]),
        "weight_stream_begin": (S, [_P, _I32]),
        "weight_stream_wait": (S, [_P, _I32, _P, ctypes.POINTER(_P)]),
        "q4_wstream_destroy": (S, [_P]),
        "q4_decode_token_streamed": (S, [_P, _P, _P]),
        "q4_decode_layer_noalloc": (S, [ctypes.POINTER(Layer), _I32, _I32, _I32, _I32, _I32,
                                        ctypes.c_float, _P, _P]),
        "q4_wstream_set_timing": (S, [_P, _I32]),
        "q4_wstream_copy_times": (S, [_P, ctypes.POINTER(ctypes.c_float),
                                      ctypes.POINTER(ctypes.c_float), _I32,
                                      ctypes.POINTER(_I32)]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise Q4Error(status, lib().q4_last_error().decode(errors="replace"))


def abi_version() -> int:
    return lib().q4_abi_version()


def _stream(stream) -> int:
    """HIP stream handle: None -> torch's current stream on the current device."""
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


# ----------------------------------------------------------------- products
def q4_pack(codes, packed, stream=None):
    N, K = codes.shape
    _check(lib().q4_pack(_ptr(codes), _ptr(packed), N, K, _stream(stream)))


def q4_unpack(packed, codes, stream=None):
    N, K = codes.shape
    _check(lib().q4_unpack(_ptr(packed), _ptr(codes), N, K, _stream(stream)))


DTYPE_F32, DTYPE_F16 = 0, 1


def q4_quantize(w, packed, scales, stream=None):
    """Quantize device weights ``w`` [N][K] (float32, or float16 / int16
    binary16 bit patterns) into ``packed`` u8[N][K/2] and ``scales``
    int16[N][K/32]."""
    N, K = w.shape
    name = str(w.dtype)
    if name.endswith("float32"):
        dt = DTYPE_F32
    elif name.endswith("float16") or name.endswith("int16"):
        dt = DTYPE_F16
    else:
        raise ValueError(f"q4_quantize: unsupported weight dtype {w.dtype}")
    _check(lib().q4_quantize(_ptr(w), dt, _ptr(packed), _ptr(scales), N, K, _stream(stream)))


def q4_gemv(packed, scales, x16, y, N=None, K=None, stream=None):
    N = packed.shape[0] if N is None else N
    K = 2 * packed.shape[1] if K is None else K
    _check(lib().q4_gemv(_ptr(packed), _ptr(scales), _ptr(x16), _ptr(y), N, K,
                         _stream(stream)))


def q4_gemm_smallbatch(packed, scales, X16, Y, B=None, N=None, K=None, stream=None):
    N = packed.shape[0] if N is None else N
    K = 2 * packed.shape[1] if K is None else K
    B = X16.shape[0] if B is None else B
    _check(lib().q4_gemm_smallbatch(_ptr(packed), _ptr(scales), _ptr(X16), _ptr(Y), N, K,
                                    B, _stream(stream)))


def q4_gemv_tuned(packed, scales, x16, y, rows_per_slot, k_split, chunks_in_flight=4,
                  nontemporal=1, stream=None):
    N, K = packed.shape[0], 2 * packed.shape[1]
    _check(lib().q4_gemv_tuned(_ptr(packed), _ptr(scales), _ptr(x16), _ptr(y), N, K,
                               rows_per_slot, k_split, chunks_in_flight, nontemporal,
                               _stream(stream)))


def q4_gemv_rows_tuned(packed, scales, x16, y, rows_per_wave, workgroups=0, stream=None):
    N, K = packed.shape[0], 2 * packed.shape[1]
    _check(lib().q4_gemv_rows_tuned(_ptr(packed), _ptr(scales), _ptr(x16), _ptr(y), N, K,
                                    rows_per_wave, workgroups, _stream(stream)))


def q4_gemv_rowp_tuned(packed, scales, x16, y, rows_per_wave, chunks_per_phase, workgroups=0,
                       stream=None):
    N, K = packed.shape[0], 2 * packed.shape[1]
    _check(lib().q4_gemv_rowp_tuned(_ptr(packed), _ptr(scales), _ptr(x16), _ptr(y), N, K,
                                    rows_per_wave, chunks_per_phase, workgroups,
                                    _stream(stream)))


def q4_gemm_valu(packed, scales, X16, Y, stream=None):
    N, K = packed.shape[0], 2 * packed.shape[1]
    B = X16.shape[0]
    _check(lib().q4_gemm_valu(_ptr(packed), _ptr(scales), _ptr(X16), _ptr(Y), N, K, B,
                              _stream(stream)))


def q4_gemm_tuned(packed, scales, X16, Y, row_tiles, waves, stream=None):
    N, K = packed.shape[0], 2 * packed.shape[1]
    B = X16.shape[0]
    _check(lib().q4_gemm_tuned(_ptr(packed), _ptr(scales), _ptr(X16), _ptr(Y), N, K, B,
                               row_tiles, waves, _stream(stream)))


# ----------------------------------------------------------------- decoder
def make_matrix(packed, scales, N=None, K=None) -> Matrix:
    N = packed.shape[0] if N is None else N
    K = 2 * packed.shape[1] if K is None else K
    return Matrix(_ptr(packed), _ptr(scales), N, K)


def make_layer(weights: dict) -> Layer:
    """weights: name -> (packed, scales) device tensors."""
    return Layer(*(make_matrix(*weights[n]) for n in ("qkv", "o", "gate_up", "down")))


def layer_shapes(dims: dict) -> Layer:
    d, H, Hkv, hd, dff = (dims[k] for k in ("d", "H", "Hkv", "hd", "dff"))
    return Layer(Matrix(0, 0, (H + 2 * Hkv) * hd, d), Matrix(0, 0, d, H * hd),
                 Matrix(0, 0, 2 * dff, d), Matrix(0, 0, d, dff))


def layer_blob_layout(dims: dict):
    """(offsets[8], total bytes) of one merged layer blob."""
    shapes = layer_shapes(dims)
    offs = (ctypes.c_size_t * 8)()
    total = ctypes.c_size_t()
    _check(lib().q4_layer_blob_layout(ctypes.byref(shapes), offs, ctypes.byref(total)))
    return list(offs), total.value


def _model_desc(dims, n_layers, layers_arr, h, workspace, ws_bytes, eps, kv_cache=None,
                max_ctx=0, rope_base=500000.0, max_batch=0, h_batch=None):
    return ModelDesc(n_layers, dims["d"], dims["H"], dims["Hkv"], dims["hd"], dims["dff"],
                     eps, layers_arr, _ptr(h), _ptr(workspace), ws_bytes, _ptr(kv_cache),
                     int(max_ctx), float(rope_base), int(max_batch), _ptr(h_batch))


def kv_cache_elems(dims: dict, n_layers: int, max_ctx: int) -> int:
    """binary16 elements of a decoder's KV cache: per layer K then V, each
    [Hkv][max_ctx][hd]."""
    return 2 * n_layers * dims["Hkv"] * max_ctx * dims["hd"]


def workspace_bytes(dims: dict, n_layers: int = None, eps: float = 1e-5,
                    max_ctx: int = 0, max_batch: int = 0) -> int:
    """Workspace bytes of a decoder; max_ctx > 0 sizes it for a KV cache of
    that many rows (the attention partials), max_batch > 0 for verify
    batches of up to that many columns."""
    n = n_layers if n_layers is not None else dims.get("n_layers", 1)
    # a non-NULL stand-in: only the sizes of a cache are read here
    desc = _model_desc(dims, n, None, 0, 0, 0, eps, 256 if max_ctx > 0 else None, max_ctx,
                       500000.0, max_batch)
    out = ctypes.c_size_t()
    _check(lib().q4_decoder_workspace_bytes(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


class Decoder:
    """Owns a q4 decoder object.  ``layers`` is a list of weight dicts (name ->
    (packed, scales)) or None for layer-by-layer use; ``h`` is the device fp32
    residual and ``workspace`` a device uint8 tensor of workspace_bytes()."""

    def __init__(self, dims: dict, layers, h, workspace, eps: float = 1e-5,
                 n_layers=None, kv_cache=None, max_ctx: int = 0,
                 rope_base: float = 500000.0, max_batch: int = 0, h_batch=None):
        self.dims = dict(dims)
        n = len(layers) if layers is not None else (n_layers or dims.get("n_layers", 1))
        arr = None
        if layers is not None:
            arr = (Layer * n)(*(make_layer(w) for w in layers))
        self._keep = (layers, h, workspace, arr, kv_cache, h_batch)  # buffers graphs bake in
        self._n_layers = n
        self._has_kv = kv_cache is not None
        desc = _model_desc(dims, n, arr, h, workspace, workspace.numel(), eps, kv_cache,
                           max_ctx, rope_base, max_batch, h_batch)
        handle = _P()
        _check(lib().q4_decoder_create(ctypes.byref(desc), ctypes.byref(handle)))
        self.handle = handle.value

    def step_graph(self, ctx_len: int, stream=None):
        _check(lib().decode_step_graph(self.handle, ctx_len, _stream(stream)))

    def set_persistent(self, mode):
        """Step implementation: False/0 four kernels per layer, True/1 the
        persistent kernel, 2 the streaming persistent kernel, 3 streaming
        workgroups with one launch per product."""
        _check(lib().q4_decoder_set_persistent(self.handle, int(mode)))

    def set_context(self, ctx_len: int, stream=None):
        """Context length of the next eager step or layer-by-layer token
        (decoders with a KV cache)."""
        _check(lib().q4_decoder_set_context(self.handle, int(ctx_len), _stream(stream)))

    def verify_eager(self, B: int, stream=None):
        """B residual columns of h_batch through all layers (verify step)."""
        _check(lib().q4_decode_verify_eager(self.handle, int(B), _stream(stream)))

    def verify_graph(self, B: int, stream=None):
        _check(lib().q4_decode_verify_graph(self.handle, int(B), _stream(stream)))

    def check(self):
        """Raise if a persistent step's grid barrier timed out (synchronous)."""
        _check(lib().q4_decoder_check(self.handle))

    def step_eager(self, stream=None):
        _check(lib().q4_decode_step_eager(self.handle, _stream(stream)))

    def step_profiled(self, stream=None):
        """Eager step; returns per-kernel durations in ms (4 per layer: QKV,
        O, gate+up, down; with a KV cache 5: QKV, attention, O, gate+up,
        down)."""
        n_layers = self._n_layers
        cap = (5 if self._has_kv else 4) * n_layers
        buf = (ctypes.c_float * cap)()
        n = _I32()
        _check(lib().q4_decode_step_profiled(self.handle, _stream(stream), buf, cap,
                                             ctypes.byref(n)))
        return list(buf[:n.value])

    def kernel_time_us(self, which: int, reps: int, stream=None) -> float:
        """Average us of kernel `which` (0 QKV, 1 O, 2 gate+up, 3 down) over
        `reps` back-to-back launches cycling through the layers.  Clobbers h."""
        out = ctypes.c_float()
        _check(lib().q4_decode_kernel_time(self.handle, which, reps, _stream(stream),
                                           ctypes.byref(out)))
        return out.value

    def layer(self, weights, stream=None):
        L = weights if isinstance(weights, Layer) else make_layer(weights)
        _check(lib().q4_decode_layer(self.handle, ctypes.byref(L), _stream(stream)))

    def layer_part(self, weights, which: int, stream=None):
        """One product of a layer: 0 QKV, 1 O, 2 gate+up, 3 down."""
        L = weights if isinstance(weights, Layer) else make_layer(weights)
        _check(lib().q4_decode_layer_part(self.handle, ctypes.byref(L), int(which),
                                          _stream(stream)))

    def token_streamed(self, ws: "WeightStream", stream=None):
        _check(lib().q4_decode_token_streamed(self.handle, ws.handle, _stream(stream)))

    def close(self):
        if getattr(self, "handle", None):
            _check(lib().q4_decoder_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def decode_layer_noalloc(weights, dims: dict, h, eps: float = 1e-5, stream=None):
    """One decoder layer on the device residual ``h`` with the library's
    static scratch array (no decoder object, no workspace, no allocation)."""
    L = weights if isinstance(weights, Layer) else make_layer(weights)
    _check(lib().q4_decode_layer_noalloc(ctypes.byref(L), dims["d"], dims["H"], dims["Hkv"],
                                         dims["hd"], dims["dff"], float(eps), _ptr(h),
                                         _stream(stream)))


def decode_step_graph(dec: Decoder, ctx_len: int, stream=None):
    dec.step_graph(ctx_len, stream)


class WeightStream:
    """Two-slot device pool fed from pinned host blobs over a copy stream."""

    def __init__(self, host_blobs, slots, copy_stream, copy2=None, chunk_bytes=0,
                 resident=None):
        """``host_blobs``: pinned host tensors per layer (None where
        ``resident`` holds the layer's device blob); ``copy2`` and
        ``chunk_bytes``: chunked transfer over two copy streams."""
        n = len(host_blobs)
        resident = resident or [None] * n
        sizes = [(b if b is not None else r) for b, r in zip(host_blobs, resident)]
        self._blob_ptrs = (_P * n)(*(_ptr(b) for b in host_blobs))
        self._blob_bytes = (ctypes.c_size_t * n)(*(t.numel() * t.element_size() for t in sizes))
        self._resident = (_P * n)(*(_ptr(r) for r in resident))
        slot_bytes = min(s.numel() * s.element_size() for s in slots)
        desc = WStreamDesc(n, self._blob_ptrs, self._blob_bytes,
                           (_P * 2)(_ptr(slots[0]), _ptr(slots[1])), slot_bytes,
                           _stream(copy_stream), _stream(copy2) if copy2 is not None else None,
                           int(chunk_bytes), self._resident)
        self._keep = (host_blobs, slots, copy_stream, copy2, resident)
        handle = _P()
        _check(lib().q4_wstream_create(ctypes.byref(desc), ctypes.byref(handle)))
        self.handle = handle.value

    def begin(self, layer: int):
        _check(lib().weight_stream_begin(self.handle, layer))

    def wait(self, layer: int, compute_stream=None) -> int:
        out = _P()
        _check(lib().weight_stream_wait(self.handle, layer, _stream(compute_stream),
                                        ctypes.byref(out)))
        return out.value

    def set_timing(self, capacity: int):
        """Record start and end events for the next `capacity` copies."""
        _check(lib().q4_wstream_set_timing(self.handle, int(capacity)))

    def copy_times(self, capacity: int):
        """(start_ms, end_ms) lists of the timed copies, relative to the
        start of the first; waits for the last one."""
        s = (ctypes.c_float * capacity)()
        e = (ctypes.c_float * capacity)()
        n = _I32()
        _check(lib().q4_wstream_copy_times(self.handle, s, e, capacity, ctypes.byref(n)))
        return list(s[:n.value]), list(e[:n.value])

    def close(self):
        if getattr(self, "handle", None):
            _check(lib().q4_wstream_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def offload_plan(n_layers: int, layer_bytes: int, budget_bytes: int):
    """Resident flags (list of 0/1) chosen by q4_offload_plan."""
    out = (_I32 * n_layers)()
    k = _I32()
    _check(lib().q4_offload_plan(n_layers, layer_bytes, budget_bytes, out, ctypes.byref(k)))
    return list(out)


def weight_stream_begin(ws: WeightStream, layer: int):
    ws.begin(layer)


def weight_stream_wait(ws: WeightStream, layer: int, compute_stream=None) -> int:
    return ws.wait(layer, compute_stream)


def layer_from_blob(dims: dict, base_ptr: int) -> Layer:
    shapes = layer_shapes(dims)
    out = Layer()
    _check(lib().q4_layer_from_blob(ctypes.byref(shapes), base_ptr, ctypes.byref(out)))
    return out
