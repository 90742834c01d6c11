"""GPU parity of the decode step (eager, graph, streamed) against the oracle.

The oracle runs the same layers free-running in fp64 from the same seeded
residual and weights, rounding to binary16 where the method stores binary16
activations.  Per element of the residual the GPU must stay within
2e-3 * M + 1e-6, where M accumulates the magnitudes sum|w x| of every product
added into that element -- the per-output bound of a single product applied to
the sum of products that forms the residual.  Graph replays, eager runs and
streamed runs must agree bitwise.
"""
import numpy as np
import pytest
import torch

import oracle
import int4_weight_streaming_q4_amd as q4
from int4_weight_streaming_q4_amd import inputs
from helpers import DEV, u16, u8

pytestmark = pytest.mark.gpu

TINY = dict(d=64, H=4, Hkv=2, hd=16, dff=96)
EPS = 1e-5


def make_layers(dims, config, n_layers, device=DEV):
    return [inputs.layer_weights(dims, config, l, device=device) for l in range(n_layers)]


def to_host(layers):
    return [{k: (u8(p), u16(s)) for k, (p, s) in L.items()} for L in layers]


def oracle_run(host_layers, dims, h0):
    h = np.asarray(h0, np.float64).copy()
    mag = np.zeros_like(h)
    out = []
    for L in host_layers:
        oracle.decode_layer(L, dims, h, mag, EPS)
        out.append((h.copy(), mag.copy()))
    return out


def check_h(h_gpu, h_ref, mag, what):
    h_gpu = np.asarray(h_gpu, np.float64)
    bound = 2e-3 * mag + 1e-6
    err = np.abs(h_gpu - h_ref)
    assert np.all(np.isfinite(h_gpu)), what
    assert np.all(err <= bound), (
        f"{what}: {int((err > bound).sum())} elements outside; worst ratio "
        f"{float((err / bound).max()):.3g}")
    rel_l2 = float(np.linalg.norm(h_gpu - h_ref) / np.linalg.norm(h_ref))
    print(f"{what}: rel L2 {rel_l2:.3g}, max err/bound {float((err / bound).max()):.3g}")
    return rel_l2


class Model:
    """Decoder plus the device buffers it retains."""

    def __init__(self, dims, layers, resident=True):
        self.dims = dims
        self.h = torch.zeros(dims["d"], dtype=torch.float32, device=DEV)
        self.ws = torch.zeros(q4.workspace_bytes(dims, n_layers=len(layers)), dtype=torch.uint8,
                              device=DEV)
        self.dec = q4.Decoder(dims, layers if resident else None, self.h, self.ws, EPS,
                              n_layers=len(layers))

    def set_h(self, h0):
        self.h.copy_(torch.as_tensor(h0, dtype=torch.float32, device=DEV))

    def workspace_sections(self, with_norm=False):
        d = self.dims
        a = lambda n: (n + 255) // 256 * 256
        o1 = a(max(d["d"], d["dff"]) * 2)
        nqkv = (d["H"] + 2 * d["Hkv"]) * d["hd"]
        o2 = o1 + a(nqkv * 4)
        o3 = o2 + a(d["H"] * d["hd"] * 2)
        ws = self.ws.cpu()
        qkv = ws[o1:o1 + nqkv * 4].view(torch.float32).numpy()
        oin = ws[o2:o2 + d["H"] * d["hd"] * 2].view(torch.int16).numpy().view(np.uint16)
        mlp = ws[o3:o3 + d["dff"] * 2].view(torch.int16).numpy().view(np.uint16)
        if with_norm:
            a16 = ws[:d["d"] * 2].view(torch.int16).numpy().view(np.uint16)
            return qkv, oin, mlp, a16
        return qkv, oin, mlp


def f16_ulp(v):
    """Spacing of binary16 values at |v| (2^-24 below the normal range)."""
    a = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(a)) - 10)


def teacher_forced_layer(m, L_dev, L_host, what, s):
    """Runs one layer product by product and checks each against the oracle
    computed from the GPU's own inputs to that product (the product bound),
    and each glue step against its definition from the GPU's fp32 values:
    V gather exact, RMSNorm within 1 binary16 ulp, SiLU gate within the
    propagated product bound plus 1 ulp."""
    d = m.dims
    H, Hkv, hd, dff = d["H"], d["Hkv"], d["hd"], d["dff"]
    s.synchronize()  # earlier layers may still be in flight on s
    h_in = m.h.cpu().numpy().astype(np.float64)
    # QKV from the normed residual
    m.dec.layer_part(L_dev, 0, s)
    s.synchronize()
    qkv, oin, _ = m.workspace_sections()
    q_ref, q_mag = oracle.gemv(*L_host["qkv"], oracle.rmsnorm_f16(h_in, EPS))
    assert oracle.within_bound(qkv, q_ref, q_mag).all(), f"{what}: QKV product"
    assert np.array_equal(oin, oracle.gqa_gather_f16(qkv.astype(np.float64), H, Hkv, hd)), \
        f"{what}: V gather is not the binary16 rounding of the GPU's V rows"
    # O, residual add
    m.dec.layer_part(L_dev, 1, s)
    s.synchronize()
    h_mid = m.h.cpu().numpy().astype(np.float64)
    o_ref, o_mag = oracle.gemv(*L_host["o"], oin)
    ref = h_in + o_ref
    assert np.all(np.abs(h_mid - ref) <= 2e-3 * o_mag + 1e-6 + np.abs(ref) * 2.0 ** -23), \
        f"{what}: O product + residual"
    # gate+up from the second norm, SiLU gate
    m.dec.layer_part(L_dev, 2, s)
    s.synchronize()
    _, _, mlp, a16 = m.workspace_sections(with_norm=True)
    a_ref = oracle.rmsnorm_f16(h_mid, EPS)
    got, want = oracle.f16_to_f64(a16), oracle.f16_to_f64(a_ref)
    assert np.all(np.abs(got - want) <= f16_ulp(want)), f"{what}: second RMSNorm"
    g_ref, g_mag = oracle.gemv(*L_host["gate_up"], a16)
    g, u = g_ref[:dff], g_ref[dff:]
    dg, du = 2e-3 * g_mag[:dff] + 1e-6, 2e-3 * g_mag[dff:] + 1e-6
    silu = g / (1.0 + np.exp(-g))
    want = silu * u
    # |silu'| <= 1.1 everywhere
    bound = 1.1 * dg * (np.abs(u) + du) + np.abs(silu) * du + f16_ulp(want)
    got = oracle.f16_to_f64(mlp)
    assert np.all(np.abs(got - want) <= bound), f"{what}: SiLU gate"
    # down, residual add
    m.dec.layer_part(L_dev, 3, s)
    s.synchronize()
    h_out = m.h.cpu().numpy().astype(np.float64)
    d_ref, d_mag = oracle.gemv(*L_host["down"], mlp)
    ref = h_mid + d_ref
    assert np.all(np.abs(h_out - ref) <= 2e-3 * d_mag + 1e-6 + np.abs(ref) * 2.0 ** -23), \
        f"{what}: down product + residual"


def test_tiny_eager_layers_match_oracle():
    n = 5
    layers = make_layers(TINY, 90, n)
    host = to_host(layers)
    h0 = inputs.residual_f32(TINY["d"], inputs.seed_of(90, 0, 9))
    ref = oracle_run(host, TINY, h0.numpy())
    m = Model(TINY, layers, resident=False)
    m.set_h(h0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for l in range(n):
            m.dec.layer(layers[l], s)
            s.synchronize()
            check_h(m.h.cpu().numpy(), ref[l][0], ref[l][1], f"tiny layer {l}")
            if l == 0:
                # glue of layer 0, checked from the oracle's own layer-0 values
                qkv, oin, _ = m.workspace_sections()
                a = oracle.rmsnorm_f16(h0.numpy().astype(np.float64), EPS)
                q_ref, q_mag = oracle.gemv(*host[0]["qkv"], a)
                assert np.all(np.abs(qkv - q_ref) <= 2e-3 * q_mag + 1e-6)
                V = q_ref[(TINY["H"] + TINY["Hkv"]) * TINY["hd"]:]
                Vm = q_mag[(TINY["H"] + TINY["Hkv"]) * TINY["hd"]:]
                grp = TINY["H"] // TINY["Hkv"]
                idx = np.array([(j // (TINY["hd"] * grp)) * TINY["hd"] + j % TINY["hd"]
                                for j in range(TINY["H"] * TINY["hd"])])
                got = oracle.f16_to_f64(oin)
                ulp = np.abs(V[idx]) * 2.0 ** -10 + 2.0 ** -24
                assert np.all(np.abs(got - V[idx]) <= 2e-3 * Vm[idx] + 1e-6 + ulp)


@pytest.mark.parametrize("persistent", [True, False])
def test_tiny_graph_equals_eager_all_buckets(persistent):
    n = 3
    layers = make_layers(TINY, 91, n)
    h0 = inputs.residual_f32(TINY["d"], inputs.seed_of(91, 0, 9))
    m = Model(TINY, layers)
    m.dec.set_persistent(persistent)
    s = torch.cuda.Stream()
    m.set_h(h0)
    torch.cuda.synchronize()
    m.dec.step_eager(s)
    s.synchronize()
    h_eager = m.h.cpu().clone()
    host = to_host(layers)
    ref = oracle_run(host, TINY, h0.numpy())
    check_h(h_eager.numpy(), ref[-1][0], ref[-1][1], "tiny eager step")
    for ctx in (1, 512, 513, 1024, 1500, 2048, 4096, 7, 4000):
        for rep in range(2):
            m.set_h(h0)
            torch.cuda.synchronize()
            m.dec.step_graph(ctx, s)
            s.synchronize()
            assert torch.equal(m.h.cpu(), h_eager), (ctx, rep)
    m.dec.check()
    with pytest.raises(q4.Q4Error, match="UNSUPPORTED"):
        m.dec.step_graph(4097, s)
    with pytest.raises(q4.Q4Error, match="INVALID_ARG"):
        m.dec.step_graph(0, s)


@pytest.mark.parametrize("persistent", [True, False])
def test_tiny_token_loop_graph_replays(persistent):
    """Several tokens through one captured graph, fed a new residual each
    token, equal to the oracle token by token."""
    n = 4
    layers = make_layers(TINY, 92, n)
    host = to_host(layers)
    m = Model(TINY, layers)
    m.dec.set_persistent(persistent)
    s = torch.cuda.Stream()
    for t in range(4):
        h0 = inputs.residual_f32(TINY["d"], inputs.seed_of(92, t, 9))
        with torch.cuda.stream(s):
            m.h.copy_(h0.to(DEV, non_blocking=False))
            m.dec.step_graph(600, s)
        s.synchronize()
        ref = oracle_run(host, TINY, h0.numpy())
        check_h(m.h.cpu().numpy(), ref[-1][0], ref[-1][1], f"tiny token {t}")
    m.dec.check()


# Small model whose widths are multiples of 64 (the streaming step's need).
SMALL = dict(d=256, H=4, Hkv=2, hd=64, dff=384)


def test_streaming_step_unsupported_shapes():
    layers = make_layers(TINY, 93, 1)
    m = Model(TINY, layers)
    with pytest.raises(q4.Q4Error, match="UNSUPPORTED"):
        m.dec.set_persistent(2)  # dff = 96 is not a multiple of 64
    with pytest.raises(q4.Q4Error, match="UNSUPPORTED"):
        m.dec.set_persistent(3)
    with pytest.raises(q4.Q4Error, match="INVALID_ARG"):
        m.dec.set_persistent(4)


@pytest.mark.parametrize("mode", [2, 3])
@pytest.mark.parametrize("n_layers", [1, 3])
def test_streaming_step_small_matches_oracle(n_layers, mode):
    """Streaming persistent step on a small model: eager against the oracle,
    graph replays over every bucket bitwise equal to eager, a token loop
    through one graph against the oracle token by token."""
    layers = make_layers(SMALL, 94, n_layers)
    host = to_host(layers)
    m = Model(SMALL, layers)
    m.dec.set_persistent(mode)
    s = torch.cuda.Stream()
    h0 = inputs.residual_f32(SMALL["d"], inputs.seed_of(94, 0, 9))
    m.set_h(h0)
    torch.cuda.synchronize()
    m.dec.step_eager(s)
    s.synchronize()
    m.dec.check()
    h_eager = m.h.cpu().clone()
    ref = oracle_run(host, SMALL, h0.numpy())
    check_h(h_eager.numpy(), ref[-1][0], ref[-1][1], f"small streaming mode {mode}, {n_layers} layers")
    for ctx in (1, 700, 2048, 4096):
        for rep in range(2):
            m.set_h(h0)
            torch.cuda.synchronize()
            m.dec.step_graph(ctx, s)
            s.synchronize()
            m.dec.check()
            assert torch.equal(m.h.cpu(), h_eager), (ctx, rep)
    for t in range(1, 4):
        h0 = inputs.residual_f32(SMALL["d"], inputs.seed_of(94, t, 9))
        with torch.cuda.stream(s):
            m.h.copy_(h0.to(DEV, non_blocking=False))
            m.dec.step_graph(600, s)
        s.synchronize()
        m.dec.check()
        ref = oracle_run(host, SMALL, h0.numpy())
        check_h(m.h.cpu().numpy(), ref[-1][0], ref[-1][1], f"small streaming token {t}")


def _big(dims_name, config, n_layers):
    dims = {k: v for k, v in inputs.MODEL_DIMS[dims_name].items() if k != "n_layers"}
    layers = make_layers(dims, config, n_layers)
    return dims, layers


def test_8b_full_step_graph_matches_oracle():
    """Llama-3-8B shapes, all 32 layers, graph-captured (four kernels per
    layer, the default step), token 0, against the oracle; graph == eager
    bitwise for both step implementations, and the persistent kernel (its
    own fixed launch shape, so its own summation order) within the same
    bound."""
    dims, layers = _big("8b", 2, 32)
    h0 = inputs.residual_f32(dims["d"], inputs.seed_of(2, 0, 9))
    m = Model(dims, layers)
    s = torch.cuda.Stream()
    m.set_h(h0)
    torch.cuda.synchronize()
    m.dec.step_graph(512, s)
    s.synchronize()
    m.dec.check()
    h_graph = m.h.cpu().clone()
    m.set_h(h0)
    torch.cuda.synchronize()
    m.dec.step_eager(s)
    s.synchronize()
    assert torch.equal(m.h.cpu(), h_graph), "graph and eager differ"
    outs = {}
    for mode in (1, 2, 3):
        m.dec.set_persistent(mode)
        got = []
        for step in (lambda: m.dec.step_eager(s), lambda: m.dec.step_graph(512, s),
                     lambda: m.dec.step_graph(512, s)):
            m.set_h(h0)
            torch.cuda.synchronize()
            step()
            s.synchronize()
            m.dec.check()
            got.append(m.h.cpu().clone())
        assert torch.equal(got[0], got[1]) and torch.equal(got[0], got[2]), \
            f"mode {mode}: graph and eager differ"
        outs[mode] = got[0]
    host = to_host(layers)
    del layers
    ref = oracle_run(host, dims, h0.numpy())
    rel = check_h(h_graph.numpy(), ref[-1][0], ref[-1][1], "8b 32 layers")
    assert rel < 1e-2
    for mode, h in outs.items():
        rel = check_h(h.numpy(), ref[-1][0], ref[-1][1], f"8b 32 layers step mode {mode}")
        assert rel < 1e-2


def test_8b_teacher_forced_all_layers():
    """Llama-3-8B shapes, tokens 0 and 255, every product of all 32 layers
    checked from the GPU's own inputs (no error accumulates between
    products); the per-layer products equal the graph step bitwise."""
    dims, layers = _big("8b", 2, 32)
    host = to_host(layers)
    m = Model(dims, layers)
    s = torch.cuda.Stream()
    for t in (0, 255):
        h0 = inputs.residual_f32(dims["d"], inputs.seed_of(2, t, 9))
        m.set_h(h0)
        torch.cuda.synchronize()
        for l in range(32):
            teacher_forced_layer(m, layers[l], host[l], f"token {t} layer {l}", s)
        h_parts = m.h.cpu().clone()
        m.set_h(h0)
        torch.cuda.synchronize()
        m.dec.step_graph(512, s)
        s.synchronize()
        assert torch.equal(m.h.cpu(), h_parts), t


def test_70b_first_layers_and_full_graph():
    """Llama-3-70B shapes: layers 0-1 against the oracle through both step
    implementations, then the full 80-layer model (about 38.5 GB resident):
    graph == eager, finite, persistent within the bound of the per-layer
    kernels' result."""
    dims = {k: v for k, v in inputs.MODEL_DIMS["70b"].items() if k != "n_layers"}
    layers = make_layers(dims, 4, 80)
    h0 = inputs.residual_f32(dims["d"], inputs.seed_of(4, 0, 9))
    s = torch.cuda.Stream()
    host2 = to_host(layers[:2])
    ref = oracle_run(host2, dims, h0.numpy())
    # two layers, eagerly per layer
    m2 = Model(dims, layers[:2], resident=False)
    m2.set_h(h0)
    torch.cuda.synchronize()
    for l in range(2):
        m2.dec.layer(layers[l], s)
    s.synchronize()
    check_h(m2.h.cpu().numpy(), ref[-1][0], ref[-1][1], "70b layers 0-1 per-layer kernels")
    # the same two layers through both persistent kernels
    m3 = Model(dims, layers[:2])
    for mode in (1, 2, 3):
        m3.dec.set_persistent(mode)
        m3.set_h(h0)
        torch.cuda.synchronize()
        m3.dec.step_eager(s)
        s.synchronize()
        m3.dec.check()
        check_h(m3.h.cpu().numpy(), ref[-1][0], ref[-1][1], f"70b layers 0-1 step mode {mode}")
    # full model
    m = Model(dims, layers)
    m.set_h(h0)
    torch.cuda.synchronize()
    m.dec.step_graph(2048, s)
    s.synchronize()
    m.dec.check()
    h_graph = m.h.cpu().clone()
    assert torch.isfinite(h_graph).all()
    m.set_h(h0)
    torch.cuda.synchronize()
    m.dec.step_eager(s)
    s.synchronize()
    assert torch.equal(m.h.cpu(), h_graph)
    # teacher-forced products of layers 0, 39 and 79
    m.set_h(h0)
    torch.cuda.synchronize()
    checked = {0, 39, 79}
    host_c = {l: to_host([layers[l]])[0] for l in checked}
    for l in range(80):
        if l in checked:
            teacher_forced_layer(m, layers[l], host_c[l], f"70b layer {l}", s)
        else:
            m.dec.layer(layers[l], s)
    s.synchronize()
    assert torch.equal(m.h.cpu(), h_graph)
