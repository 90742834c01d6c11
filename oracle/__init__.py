"""CPU oracle for the INT4 weight-streaming decode path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding in ``int4_weight_streaming_q4_amd``) never imports it, and the two
share no code: the oracle is plain single-threaded fp64 C in ``q4_oracle.c``,
loaded here through ctypes, with numpy arrays at the boundary.

What each function computes, and which passage it follows, is documented next
to its C definition.  The pins that tie it to something other than itself are
in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4_oracle.c")
_LIB = os.path.join(_HERE, "libq4oracle.so")
_LIB_OMP = os.path.join(_HERE, "libq4oracle_omp.so")

# No fast-math and no contraction: every product and sum rounds once, in the
# order the source states.  The oracle is single-threaded (its one OpenMP
# pragma is ignored without -fopenmp).
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unknown-pragmas"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (and its all-core baseline build);
    returns the oracle's library path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    build_omp(force)
    return _LIB


def build_omp(force: bool = True) -> str:
    """The same source with -fopenmp: the all-core CPU baseline (product rows
    split over threads).  Not the oracle; only the benchmark's CPU-baseline
    leg loads it."""
    if force or not os.path.exists(_LIB_OMP):
        tmp = _LIB_OMP + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-fopenmp", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_OMP)
    return _LIB_OMP


_lib = None
_lib_omp = None


def lib(all_cores: bool = False) -> ctypes.CDLL:
    """The oracle library; all_cores=True: the OpenMP baseline build."""
    global _lib, _lib_omp
    if all_cores:
        if _lib_omp is None:
            if not os.path.exists(_LIB_OMP):
                build_omp(force=False)
            _lib_omp = _declare(ctypes.CDLL(_LIB_OMP))
        return _lib_omp
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _declare(L: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.c_void_p
    I = ctypes.c_int64
    D = ctypes.c_double
    L.q4o_f16_to_f64.restype = D
    L.q4o_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.q4o_f64_to_f16.restype = ctypes.c_uint16
    L.q4o_f64_to_f16.argtypes = [D]
    for name, args in {
        "q4o_f16_to_f64_array": [P, P, I],
        "q4o_f64_to_f16_array": [P, P, I],
        "q4o_pack": [P, P, I, I],
        "q4o_unpack": [P, P, I, I],
        "q4o_dequant": [P, P, P, I, I],
        "q4o_gemv": [P, P, P, I, I, P, P],
        "q4o_gemv_rows": [P, P, P, I, P, I, P, P],
        "q4o_gemm": [P, P, P, I, I, I, P, P],
        "q4o_rmsnorm_f16": [P, I, D, P],
        "q4o_gqa_gather_f16": [P, I, I, I, P],
        "q4o_silu_mul_f16": [P, I, P],
        "q4o_decode_layer": [P, P, P, P, I, I, I, I, I, D, P, P],
        "q4o_rope": [P, I, I, D],
        "q4o_attention": [P, I, I, I, I, I, D, P, P, P, P],
        "q4o_decode_layer_attn": [P, P, P, P, I, I, I, I, I, D, I, I, D, P, P, P, P],
        "q4o_quantize_f32": [P, I, I, P, P],
        "q4o_quantize_f16": [P, I, I, P, P],
    }.items():
        fn = getattr(L, name)
        fn.restype = None
        fn.argtypes = args
    return L


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


# ---------------------------------------------------------------- binary16
def f16_to_f64(h) -> np.ndarray:
    """binary16 bit patterns (uint16) -> float64, decoded by hand."""
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().q4o_f16_to_f64_array(_ptr(h), _ptr(out), h.size)
    return out


def f64_to_f16(v) -> np.ndarray:
    """float64 -> binary16 bit patterns, round to nearest even."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().q4o_f64_to_f16_array(_ptr(v), _ptr(out), v.size)
    return out


# ---------------------------------------------------------------- packing
def pack(codes) -> np.ndarray:
    """codes u8[N][K] -> packed u8[N][K/2] (low nibble = even k)."""
    codes = _c(codes, np.uint8)
    N, K = codes.shape
    assert K % 2 == 0
    out = np.empty((N, K // 2), np.uint8)
    lib().q4o_pack(_ptr(codes), _ptr(out), N, K)
    return out


def unpack(packed) -> np.ndarray:
    packed = _c(packed, np.uint8)
    N, K2 = packed.shape
    out = np.empty((N, 2 * K2), np.uint8)
    lib().q4o_unpack(_ptr(packed), _ptr(out), N, 2 * K2)
    return out


def dequant(packed, scales) -> np.ndarray:
    """Dense fp64 W[N][K]; small matrices only."""
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint16)
    N, K2 = packed.shape
    K = 2 * K2
    assert scales.shape == (N, K // 32)
    W = np.empty((N, K), np.float64)
    lib().q4o_dequant(_ptr(packed), _ptr(scales), _ptr(W), N, K)
    return W


# ---------------------------------------------------------------- products
def _check_mat(packed, scales):
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint16)
    N, K2 = packed.shape
    K = 2 * K2
    assert K % 32 == 0 and scales.shape == (N, K // 32), (packed.shape, scales.shape)
    return packed, scales, N, K


def gemv(packed, scales, x_f16, all_cores=False):
    """(y, mag): y[n] = sum_k w[n][k] x[k], mag[n] = sum_k |w[n][k] x[k]|.
    all_cores: the OpenMP baseline build (same result, rows in parallel)."""
    packed, scales, N, K = _check_mat(packed, scales)
    x = _c(x_f16, np.uint16)
    assert x.shape == (K,)
    y = np.empty(N, np.float64)
    m = np.empty(N, np.float64)
    lib(all_cores).q4o_gemv(_ptr(packed), _ptr(scales), _ptr(x), N, K, _ptr(y), _ptr(m))
    return y, m


def gemv_rows(packed, scales, x_f16, rows):
    """gemv restricted to the given row indices."""
    packed, scales, N, K = _check_mat(packed, scales)
    x = _c(x_f16, np.uint16)
    rows = _c(rows, np.int64)
    assert x.shape == (K,) and (rows.size == 0 or (rows.min() >= 0 and rows.max() < N))
    y = np.empty(rows.size, np.float64)
    m = np.empty(rows.size, np.float64)
    lib().q4o_gemv_rows(_ptr(packed), _ptr(scales), _ptr(x), K, _ptr(rows),
                        rows.size, _ptr(y), _ptr(m))
    return y, m


def gemm(packed, scales, X_f16):
    """(Y, M) with Y[b][n] = sum_k w[n][k] X[b][k]."""
    packed, scales, N, K = _check_mat(packed, scales)
    X = _c(X_f16, np.uint16)
    B = X.shape[0]
    assert X.shape == (B, K)
    Y = np.empty((B, N), np.float64)
    M = np.empty((B, N), np.float64)
    lib().q4o_gemm(_ptr(packed), _ptr(scales), _ptr(X), N, K, B, _ptr(Y), _ptr(M))
    return Y, M


def within_bound(y, y_ref, mag, rel=2e-3, abs_=1e-6):
    """The per-output acceptance rule |y - y_ref| <= rel*mag + abs."""
    y = np.asarray(y, np.float64)
    return np.abs(y - y_ref) <= rel * np.asarray(mag) + abs_


# ---------------------------------------------------------------- glue
def rmsnorm_f16(h, eps=1e-5) -> np.ndarray:
    h = _c(h, np.float64)
    out = np.empty(h.shape, np.uint16)
    lib().q4o_rmsnorm_f16(_ptr(h), h.size, eps, _ptr(out))
    return out


def gqa_gather_f16(qkv, H, Hkv, hd) -> np.ndarray:
    qkv = _c(qkv, np.float64)
    assert qkv.size == (H + 2 * Hkv) * hd and H % Hkv == 0
    out = np.empty(H * hd, np.uint16)
    lib().q4o_gqa_gather_f16(_ptr(qkv), H, Hkv, hd, _ptr(out))
    return out


def silu_mul_f16(gu) -> np.ndarray:
    gu = _c(gu, np.float64)
    assert gu.size % 2 == 0
    dff = gu.size // 2
    out = np.empty(dff, np.uint16)
    lib().q4o_silu_mul_f16(_ptr(gu), dff, _ptr(out))
    return out


def rope(x, pos, base=500000.0) -> np.ndarray:
    """Rotate-half rotary embedding of one head vector at position pos."""
    x = np.array(x, np.float64, copy=True, order="C")
    assert x.ndim == 1 and x.size % 2 == 0
    lib().q4o_rope(_ptr(x), x.size, pos, base)
    return x


def kv_cache(dims, max_ctx):
    """Empty binary16 K and V caches of one layer, [Hkv][max_ctx][hd]."""
    shape = (dims["Hkv"], max_ctx, dims["hd"])
    return np.zeros(shape, np.uint16), np.zeros(shape, np.uint16)


def attention(qkv, dims, pos, kcache, vcache, base=500000.0):
    """Decode attention at position pos (writes row pos of both caches).
    Returns (o, mag): fp64 [H*hd] output and sum_j p_j |v_j|."""
    H, Hkv, hd = dims["H"], dims["Hkv"], dims["hd"]
    qkv = _c(qkv, np.float64)
    assert qkv.size == (H + 2 * Hkv) * hd and H % Hkv == 0
    assert kcache.dtype == np.uint16 and vcache.dtype == np.uint16
    assert kcache.flags["C_CONTIGUOUS"] and vcache.flags["C_CONTIGUOUS"]
    assert kcache.shape == vcache.shape and kcache.shape[0] == Hkv and kcache.shape[2] == hd
    max_ctx = kcache.shape[1]
    assert 0 <= pos < max_ctx
    out = np.empty(H * hd, np.float64)
    mag = np.empty(H * hd, np.float64)
    lib().q4o_attention(_ptr(qkv), H, Hkv, hd, pos, max_ctx, base, _ptr(kcache),
                        _ptr(vcache), _ptr(out), _ptr(mag))
    return out, mag


def quantize(w):
    """Symmetric round-to-nearest per group of 32 (see q4o_quantize_f32).
    ``w``: float32 [N][K], or binary16 bit patterns as uint16 [N][K].
    Returns (codes u8[N][K], scales u16[N][K/32])."""
    w = np.asarray(w)
    assert w.ndim == 2 and w.shape[1] % 32 == 0
    N, K = w.shape
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((N, K // 32), np.uint16)
    if w.dtype == np.uint16:
        w = np.ascontiguousarray(w)
        lib().q4o_quantize_f16(_ptr(w), N, K, _ptr(codes), _ptr(scales))
    else:
        assert w.dtype == np.float32, w.dtype
        w = np.ascontiguousarray(w)
        lib().q4o_quantize_f32(_ptr(w), N, K, _ptr(codes), _ptr(scales))
    return codes, scales


class _Mat(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


def decode_layer(layer, dims, h, mag_h=None, eps=1e-5, all_cores=False):
    """Run one decoder layer in place on the fp64 residual ``h``.

    ``layer`` maps "qkv", "o", "gate_up", "down" to (packed, scales) numpy
    pairs; ``dims`` is a dict with d, H, Hkv, hd, dff.  ``mag_h``, if given,
    accumulates the magnitude sums of the two products added into h.
    """
    d, H, Hkv, hd, dff = (dims[k] for k in ("d", "H", "Hkv", "hd", "dff"))
    shapes = {"qkv": ((H + 2 * Hkv) * hd, d), "o": (d, H * hd),
              "gate_up": (2 * dff, d), "down": (d, dff)}
    keep = []
    mats = []
    for name in ("qkv", "o", "gate_up", "down"):
        p, s, N, K = _check_mat(*layer[name])
        assert (N, K) == shapes[name], (name, (N, K), shapes[name])
        keep += [p, s]
        mats.append(_Mat(p.ctypes.data, s.ctypes.data))
    assert h.dtype == np.float64 and h.flags["C_CONTIGUOUS"] and h.shape == (d,)
    if mag_h is not None:
        assert mag_h.dtype == np.float64 and mag_h.shape == (d,)
    lib(all_cores).q4o_decode_layer(*(ctypes.addressof(m) for m in mats), d, H, Hkv, hd,
                                    dff, eps, _ptr(h),
                                    _ptr(mag_h) if mag_h is not None else None)
    return h


def decode_layer_attn(layer, dims, h, pos, kcache, vcache, mag_h=None, eps=1e-5,
                      base=500000.0):
    """decode_layer with attention over this layer's caches at position pos
    (row pos of both caches is written)."""
    d, H, Hkv, hd, dff = (dims[k] for k in ("d", "H", "Hkv", "hd", "dff"))
    shapes = {"qkv": ((H + 2 * Hkv) * hd, d), "o": (d, H * hd),
              "gate_up": (2 * dff, d), "down": (d, dff)}
    keep = []
    mats = []
    for name in ("qkv", "o", "gate_up", "down"):
        p, s, N, K = _check_mat(*layer[name])
        assert (N, K) == shapes[name], (name, (N, K), shapes[name])
        keep += [p, s]
        mats.append(_Mat(p.ctypes.data, s.ctypes.data))
    assert h.dtype == np.float64 and h.flags["C_CONTIGUOUS"] and h.shape == (d,)
    assert kcache.shape == vcache.shape == (Hkv, kcache.shape[1], hd)
    assert kcache.dtype == vcache.dtype == np.uint16
    max_ctx = kcache.shape[1]
    assert 0 <= pos < max_ctx
    if mag_h is not None:
        assert mag_h.dtype == np.float64 and mag_h.shape == (d,)
    lib().q4o_decode_layer_attn(*(ctypes.addressof(m) for m in mats), d, H, Hkv, hd,
                                dff, eps, pos, max_ctx, base, _ptr(kcache), _ptr(vcache),
                                _ptr(h), _ptr(mag_h) if mag_h is not None else None)
    return h
