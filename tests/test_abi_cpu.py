"""C-ABI checks that need no GPU: the library loads, exports every function
include/q4.h declares, and rejects bad arguments before enqueuing anything.

Only host-side validation paths are exercised here (they return before any
HIP call); nothing below launches a kernel.
"""
import ctypes
import os
import re

import pytest

import int4_weight_streaming_q4_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]

INVALID, UNSUPPORTED, STATE = 1, 2, 4


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(
        r"^\s*(?:q4_status|const char \*|int32_t)\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    L = q4.lib()
    names = declared_functions()
    assert len(names) >= 20, names
    for n in names:
        assert hasattr(L, n), n
    assert q4.abi_version() == 5
    assert {"q4_gemv_tuned", "q4_wstream_copy_times", "q4_pack"} <= set(names)


def _err():
    return q4.lib().q4_last_error().decode()


def test_gemv_argument_checks():
    L = q4.lib()
    buf = 4096  # fake, 16-byte aligned, never dereferenced
    assert L.q4_gemv(0, buf, buf, buf, 16, 64, None) == INVALID
    assert "null" in _err()
    assert L.q4_gemv(buf, buf, buf, buf, 0, 64, None) == INVALID
    assert L.q4_gemv(buf, buf, buf, buf, 16, 48, None) == INVALID
    assert "multiple of 32" in _err()
    assert L.q4_gemv(buf, buf, buf, buf, 16, 16, None) == INVALID
    assert L.q4_gemv(buf, buf, buf, buf, 16, 65536, None) == UNSUPPORTED
    assert L.q4_gemv(buf + 8, buf, buf, buf, 16, 64, None) == INVALID
    assert "16-byte" in _err()
    assert L.q4_gemv(buf, buf + 1, buf, buf, 16, 64, None) == INVALID
    assert L.q4_gemv(buf, buf, buf + 2, buf, 16, 64, None) == INVALID
    assert L.q4_gemv(buf, buf, buf, buf + 2, 16, 64, None) == INVALID
    assert L.q4_gemv(buf, buf, buf, 0, 16, 64, None) == INVALID
    assert L.q4_gemv_tuned(buf, buf, buf, buf, 16, 64, 3, 1, 4, 1, None) == INVALID
    assert L.q4_gemv_tuned(buf, buf, buf, buf, 16, 64, 1, 8, 4, 1, None) == INVALID
    assert L.q4_gemv_tuned(buf, buf, buf, buf, 16, 64, 1, 1, 6, 1, None) == INVALID
    # the pipelined loop (two chunks in flight per buffer) needs K % (1024 *
    # k_split) == 0 and non-temporal loads; refused before anything is launched
    assert L.q4_gemv_tuned(buf, buf, buf, buf, 16, 1056, 1, 1, 2, 1, None) == UNSUPPORTED
    assert "pipelined" in _err()
    assert L.q4_gemv_tuned(buf, buf, buf, buf, 16, 1024, 1, 2, 2, 1, None) == UNSUPPORTED
    assert L.q4_gemv_tuned(buf, buf, buf, buf, 16, 1024, 1, 1, 2, 0, None) == UNSUPPORTED


def test_gemm_argument_checks():
    L = q4.lib()
    buf = 4096
    assert L.q4_gemm_smallbatch(buf, buf, buf, buf, 16, 64, 0, None) == INVALID
    assert L.q4_gemm_smallbatch(buf, buf, buf, buf, 16, 64, 17, None) == INVALID
    assert "outside [1, 16]" in _err()
    assert L.q4_gemm_smallbatch(buf, buf, buf + 4, buf, 16, 64, 4, None) == INVALID
    assert L.q4_gemm_tuned(buf, buf, buf, buf, 16, 64, 4, 3, 4, None) == UNSUPPORTED
    assert L.q4_gemm_tuned(buf, buf, buf, buf, 16, 64, 4, 8, 8, None) == UNSUPPORTED
    assert L.q4_gemm_tuned(buf, buf, buf, buf, 16, 64, 4, 4, 16, None) == UNSUPPORTED
    # vector-ALU batch kernel: B in {2, 3, 4, 8}, columns within 64 KB of LDS
    assert L.q4_gemm_valu(buf, buf, buf, buf, 16, 64, 5, None) == UNSUPPORTED
    assert L.q4_gemm_valu(buf, buf, buf, buf, 16, 64, 1, None) == UNSUPPORTED
    assert L.q4_gemm_valu(buf, buf, buf, buf, 16, 14336, 3, None) == UNSUPPORTED
    assert "LDS" in _err()
    assert L.q4_gemm_valu(buf, buf, 0, buf, 16, 64, 2, None) == INVALID
    assert L.q4_gemm_valu(buf, buf, buf + 2, buf, 16, 64, 2, None) == INVALID


def test_pack_argument_checks():
    L = q4.lib()
    assert L.q4_pack(0, 4096, 4, 8, None) == INVALID
    assert L.q4_pack(4096, 4096, 4, 7, None) == INVALID
    assert L.q4_unpack(4096, 4096, 0, 8, None) == INVALID


DIMS = dict(d=64, H=4, Hkv=2, hd=16, dff=96)


def _desc(**over):
    kw = dict(n_layers=2, d_model=64, n_heads=4, n_kv_heads=2, head_dim=16, d_ff=96,
              eps=1e-5, layers=None, h=4096, workspace=4096, workspace_bytes=1 << 20)
    kw.update(over)
    return q4.ModelDesc(**kw)


def test_decoder_workspace_and_create_checks():
    L = q4.lib()
    out = ctypes.c_size_t()
    assert L.q4_decoder_workspace_bytes(ctypes.byref(_desc()), ctypes.byref(out)) == 0
    # a16 f16[max(d, dff)], qkv f32[(H+2Hkv)hd], o_in f16[H hd], mlp f16[dff],
    # barrier area (64 + 4096 + 1 words, rounded up: 16896 bytes), device layer
    # table (2 x 64 bytes), each rounded up to 256
    assert out.value == 256 + 512 + 256 + 256 + 16896 + 256
    assert q4.workspace_bytes(DIMS, n_layers=2) == out.value
    h = ctypes.c_void_p()
    assert L.q4_decoder_create(ctypes.byref(_desc(n_heads=3)), ctypes.byref(h)) == INVALID
    assert L.q4_decoder_create(ctypes.byref(_desc(d_model=48)), ctypes.byref(h)) == INVALID
    assert L.q4_decoder_create(ctypes.byref(_desc(workspace=4100)), ctypes.byref(h)) == INVALID
    assert L.q4_decoder_create(ctypes.byref(_desc(workspace_bytes=100)),
                               ctypes.byref(h)) == INVALID
    assert L.q4_decoder_create(ctypes.byref(_desc(h=0)), ctypes.byref(h)) == INVALID
    assert L.q4_decoder_create(ctypes.byref(_desc(h=4104)), ctypes.byref(h)) == INVALID
    # a layer with a wrong shape is rejected at create
    bad = q4.layer_shapes(DIMS)
    for m in (bad.qkv, bad.o, bad.gate_up, bad.down):
        m.packed, m.scales = 4096, 4096
    bad.o.N = 32
    arr = (q4.Layer * 2)(bad, bad)
    assert L.q4_decoder_create(ctypes.byref(_desc(layers=arr)), ctypes.byref(h)) == INVALID
    assert "expected" in _err()


def test_quantize_argument_checks():
    L = q4.lib()
    ok = dict(w=4096, dt=0, p=4096, s=4096, N=4, K=64)
    def call(**over):
        a = dict(ok, **over)
        return L.q4_quantize(a["w"], a["dt"], a["p"], a["s"], a["N"], a["K"], None)
    for over in (dict(w=0), dict(p=0), dict(s=0), dict(dt=2), dict(dt=-1), dict(N=0),
                 dict(K=16), dict(K=48), dict(w=4100), dict(p=4104), dict(s=4097),
                 dict(N=1 << 41)):
        assert call(**over) == INVALID, over
    assert "q4_quantize" in _err()


def test_decoder_kv_cache_description_checks():
    """A KV cache adds a position word, the attention partials, the rotated
    queries and the rotation table to the workspace; its description is
    validated before any HIP call."""
    L = q4.lib()
    dims = dict(d=128, H=4, Hkv=2, hd=64, dff=96)
    base = dict(n_layers=2, d_model=128, n_heads=4, n_kv_heads=2, head_dim=64, d_ff=96)
    plain, with_kv = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.q4_decoder_workspace_bytes(ctypes.byref(_desc(**base)), ctypes.byref(plain)) == 0
    desc = _desc(**base, kv_cache=4096, max_ctx=100, rope_base=500000.0)
    assert L.q4_decoder_workspace_bytes(ctypes.byref(desc), ctypes.byref(with_kv)) == 0
    # position word (256) + partials H * ceil(max_ctx / 64) * (hd + 2) fp32,
    # rounded up to 256: 4 * 2 * 66 * 4 = 2112 -> 2304, + rotated queries
    # H * hd fp32: 4 * 64 * 4 = 1024, + rotation table max_ctx * hd/2
    # (cos, sin) fp32 pairs: 100 * 32 * 8 = 25600
    assert with_kv.value - plain.value == 256 + 2304 + 1024 + 25600
    assert q4.workspace_bytes(dims, n_layers=2, max_ctx=100) == with_kv.value
    assert q4.kv_cache_elems(dims, 2, 100) == 2 * 2 * 2 * 100 * 64
    out = ctypes.c_size_t()
    for over, want in ((dict(kv_cache=4100), INVALID), (dict(max_ctx=0), INVALID),
                       (dict(max_ctx=(1 << 20) + 1), INVALID),
                       (dict(rope_base=0.0), INVALID), (dict(rope_base=float("nan")), INVALID),
                       (dict(head_dim=32), UNSUPPORTED),
                       (dict(n_heads=6, d_model=192), UNSUPPORTED)):
        kw = dict(base, kv_cache=4096, max_ctx=100, rope_base=500000.0)
        kw.update(over)
        assert L.q4_decoder_workspace_bytes(ctypes.byref(_desc(**kw)), ctypes.byref(out)) \
            == want, over
    # a decoder without a cache has no context to set
    h = ctypes.c_void_p()
    assert L.q4_decoder_create(ctypes.byref(_desc()), ctypes.byref(h)) == 0
    try:
        assert L.q4_decoder_set_context(h, 1, None) == STATE
    finally:
        assert L.q4_decoder_destroy(h) == 0
    assert L.q4_decoder_set_context(None, 1, None) == INVALID


def test_decoder_verify_checks():
    """Verify-step sections: per column d f16, nqkv f32, H hd f16, dff f16
    (the gate+up product writes the gated activation directly), each
    rounded up to 256; argument and state errors before HIP."""
    L = q4.lib()
    plain, with_b = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.q4_decoder_workspace_bytes(ctypes.byref(_desc()), ctypes.byref(plain)) == 0
    assert L.q4_decoder_workspace_bytes(ctypes.byref(_desc(max_batch=9, h_batch=8192)),
                                        ctypes.byref(with_b)) == 0
    a = lambda n: (n + 255) // 256 * 256
    # DIMS: d 64, nqkv (4 + 4) * 16 = 128, H hd 64, dff 96
    want = a(9 * 64 * 2) + a(9 * 128 * 4) + a(9 * 64 * 2) + a(9 * 96 * 2)
    assert with_b.value - plain.value == want
    assert q4.workspace_bytes(DIMS, n_layers=2, max_batch=9) == with_b.value
    out = ctypes.c_size_t()
    for mb in (-1, 17):
        assert L.q4_decoder_workspace_bytes(ctypes.byref(_desc(max_batch=mb)),
                                            ctypes.byref(out)) == INVALID
    h = ctypes.c_void_p()
    big = dict(workspace_bytes=1 << 22)
    assert L.q4_decoder_create(ctypes.byref(_desc(max_batch=4, **big)), ctypes.byref(h)) == INVALID
    assert L.q4_decoder_create(ctypes.byref(_desc(max_batch=4, h_batch=8200, **big)),
                               ctypes.byref(h)) == INVALID
    assert L.q4_decoder_create(ctypes.byref(_desc(max_batch=4, h_batch=8192, **big)),
                               ctypes.byref(h)) == 0
    try:
        assert L.q4_decode_verify_eager(h, 1, None) == STATE    # no resident layers
        assert L.q4_decode_verify_graph(h, 1, None) == STATE
    finally:
        assert L.q4_decoder_destroy(h) == 0
    assert L.q4_decode_verify_eager(None, 1, None) == INVALID


def test_decoder_host_object_and_step_checks():
    """A decoder without resident layers is a host object only; graph steps
    validate ctx_len and the stream before touching HIP."""
    L = q4.lib()
    h = ctypes.c_void_p()
    assert L.q4_decoder_create(ctypes.byref(_desc()), ctypes.byref(h)) == 0
    try:
        assert L.decode_step_graph(h, 0, 1234) == INVALID
        assert L.decode_step_graph(h, -5, 1234) == INVALID
        assert L.decode_step_graph(h, 4097, 1234) == UNSUPPORTED
        assert L.decode_step_graph(h, 100, None) == INVALID  # NULL stream
        assert L.decode_step_graph(h, 100, 1234) == STATE    # no resident layers
        assert L.q4_decode_step_eager(h, None) == STATE
        assert L.q4_decode_layer(h, None, None) == INVALID
        shapes = q4.layer_shapes(DIMS)
        for which in (-1, 4):
            assert L.q4_decode_layer_part(h, ctypes.byref(shapes), which, None) == INVALID
        assert L.q4_decode_layer_part(h, None, 0, None) == INVALID
        # shapes without device pointers fail the matrix checks, before any launch
        assert L.q4_decode_layer_part(h, ctypes.byref(shapes), 0, None) == INVALID
    finally:
        assert L.q4_decoder_destroy(h) == 0
    assert L.decode_step_graph(None, 100, 1234) == INVALID


def test_noalloc_layer_checks():
    """q4_decode_layer_noalloc validates before touching the device: null
    or misaligned pointers and wrong shapes are INVALID_ARG, a layer whose
    intermediates exceed the static scratch array is UNSUPPORTED."""
    L = q4.lib()
    buf = 1 << 20

    def layer(d, H, Hkv, hd, dff):
        M = lambda N, K: q4.Matrix(buf, buf, N, K)
        return q4.Layer(M((H + 2 * Hkv) * hd, d), M(d, H * hd), M(2 * dff, d), M(d, dff))

    f = L.q4_decode_layer_noalloc
    lay = layer(64, 4, 2, 16, 96)
    assert f(None, 64, 4, 2, 16, 96, 1e-5, buf, None) == INVALID
    assert f(ctypes.byref(lay), 64, 4, 2, 16, 96, 1e-5, None, None) == INVALID
    assert f(ctypes.byref(lay), 64, 4, 2, 16, 96, 1e-5, buf + 4, None) == INVALID
    assert f(ctypes.byref(lay), 96, 4, 2, 16, 96, 1e-5, buf, None) == INVALID   # shapes
    assert f(ctypes.byref(lay), 64, 4, 3, 16, 96, 1e-5, buf, None) == INVALID   # H % Hkv
    big = layer(32768, 256, 8, 128, 32768)   # 335,872 scratch bytes > 262,144
    assert f(ctypes.byref(big), 32768, 256, 8, 128, 32768, 1e-5, buf, None) == UNSUPPORTED
    assert "scratch" in _err()


def test_blob_layout_is_aligned_and_ordered():
    offs, total = q4.layer_blob_layout(DIMS)
    sizes = [(128 * 64) // 2, 128 * 2 * 2, 64 * 64 // 2, 64 * 2 * 2,
             192 * 64 // 2, 192 * 2 * 2, 64 * 96 // 2, 64 * 3 * 2]
    assert offs[0] == 0
    for i in range(8):
        assert offs[i] % 256 == 0
        end = offs[i] + sizes[i]
        nxt = offs[i + 1] if i < 7 else total
        assert end <= nxt < end + 256
    # 8B shapes: the merged blob is the four matrices plus scales, padded
    dims8 = dict(d=4096, H=32, Hkv=8, hd=128, dff=14336)
    _, total8 = q4.layer_blob_layout(dims8)
    assert 122683392 <= total8 < 122683392 + 8 * 256
    layer = q4.layer_from_blob(DIMS, 1 << 20)
    assert layer.o.packed == (1 << 20) + offs[2] and layer.down.scales == (1 << 20) + offs[7]


def test_wstream_argument_checks():
    L = q4.lib()
    out = ctypes.c_void_p()
    blobs = (ctypes.c_void_p * 2)(4096, 8192)
    sizes = (ctypes.c_size_t * 2)(1000, 5000)
    d = q4.WStreamDesc(2, blobs, sizes, (ctypes.c_void_p * 2)(4096, 8192), 4096, 1234)
    assert L.q4_wstream_create(ctypes.byref(d), ctypes.byref(out)) == INVALID  # 5000 > slot
    assert "larger than a slot" in _err()
    d2 = q4.WStreamDesc(2, blobs, sizes, (ctypes.c_void_p * 2)(4096, 0), 8192, 1234)
    assert L.q4_wstream_create(ctypes.byref(d2), ctypes.byref(out)) == INVALID
    d3 = q4.WStreamDesc(0, blobs, sizes, (ctypes.c_void_p * 2)(4096, 8192), 8192, 1234)
    assert L.q4_wstream_create(ctypes.byref(d3), ctypes.byref(out)) == INVALID
    d4 = q4.WStreamDesc(2, blobs, sizes, (ctypes.c_void_p * 2)(4096, 8192), 8192, None)
    assert L.q4_wstream_create(ctypes.byref(d4), ctypes.byref(out)) == INVALID
    # chunked transfer: pieces of a multiple of 256 bytes
    d5 = q4.WStreamDesc(2, blobs, sizes, (ctypes.c_void_p * 2)(4096, 8192), 8192, 1234, 5678,
                        100, None)
    assert L.q4_wstream_create(ctypes.byref(d5), ctypes.byref(out)) == INVALID
    assert "multiple of 256" in _err()
    # a resident blob must be 256-byte aligned; a resident layer needs no host blob
    res = (ctypes.c_void_p * 2)(4096 + 16, None)
    d6 = q4.WStreamDesc(2, (ctypes.c_void_p * 2)(None, 8192), sizes,
                        (ctypes.c_void_p * 2)(4096, 8192), 8192, 1234, None, 0, res)
    assert L.q4_wstream_create(ctypes.byref(d6), ctypes.byref(out)) == INVALID
    assert "aligned" in _err()
    assert L.weight_stream_begin(None, 0) == INVALID
    slot = ctypes.c_void_p()
    assert L.weight_stream_wait(None, 0, None, ctypes.byref(slot)) == INVALID


def test_offload_plan():
    """Placement for partial residency: everything resident when it fits;
    else the budget minus two streaming slots, spread evenly; too small a
    budget is UNSUPPORTED."""
    LB = 481_296_384                     # 70B layer blob
    assert q4.offload_plan(80, LB, 80 * LB) == [1] * 80
    assert q4.offload_plan(80, LB, 200 * LB) == [1] * 80
    flags = q4.offload_plan(80, LB, 2 * LB)
    assert flags == [0] * 80             # only the two slots fit
    for budget_layers in (3, 10, 42, 79):
        flags = q4.offload_plan(80, LB, budget_layers * LB + LB // 2)
        k = budget_layers - 2
        assert sum(flags) == k
        idx = [i for i, f in enumerate(flags) if f]
        assert idx == [(2 * i + 1) * 80 // (2 * k) for i in range(k)]
        gaps = [b - a for a, b in zip(idx, idx[1:])]
        assert not gaps or max(gaps) - min(gaps) <= 1       # evenly spread
        assert (k + 2) * LB <= budget_layers * LB + LB // 2  # within the budget
    assert q4.offload_plan(1, LB, LB) == [1]
    flags = q4.offload_plan(5, 10, 49)   # 4 fit after nothing else: 4 - 2 = 2 resident
    assert sum(flags) == 2
    L = q4.lib()
    arr = (ctypes.c_int32 * 4)()
    k = ctypes.c_int32()
    assert L.q4_offload_plan(4, 100, 150, arr, ctypes.byref(k)) == UNSUPPORTED
    assert L.q4_offload_plan(0, 100, 150, arr, ctypes.byref(k)) == INVALID
    assert L.q4_offload_plan(4, 0, 150, arr, ctypes.byref(k)) == INVALID


def test_plain_c_consumer(tmp_path):
    """The C ABI used from a plain C program (gcc, include/q4.h, linked to
    libq4stream.so): no Python or torch types cross the boundary."""
    import shutil
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = os.path.join(root, "tests", "c", "abi_host_check.c")
    libdir = os.path.dirname(q4.LIB_PATH)
    exe = str(tmp_path / "abi_host_check")
    subprocess.run([gcc, "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"),
                    "-I", "/opt/rocm/include", src, "-o", exe, "-L", libdir, "-lq4stream",
                    f"-Wl,-rpath,{libdir}"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "passed" in r.stdout


def test_bench_refuses_several_gpus():
    """The measurement script runs on one GPU: asking for more exits with
    status 2 and says so, before touching any device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
