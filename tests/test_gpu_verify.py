"""GPU parity of the batched verify step (B token columns through every
layer together, products as small-batch INT4 products) against the oracle.

A causal batch gives each column exactly the result of decoding its token
alone, so the oracle is the plain per-token layer loop, run free from each
column's seeded residual.  Per residual element the GPU must stay within
2e-3 * M + 1e-6, M the magnitudes sum|w x| of all products added into the
element (the decode tests' bound).  Graph replays equal eager bitwise; B = 1
equals the single-token step bitwise; a column's result does not depend on
B or on the other columns (bitwise)."""
import numpy as np
import pytest
import torch

import oracle
import int4_weight_streaming_q4_amd as q4
from int4_weight_streaming_q4_amd import inputs
from helpers import DEV, u16
from test_gpu_decode import SMALL, TINY, EPS, check_h, make_layers, oracle_run, to_host
from test_gpu_attention import BASE, VARIANTS, f16_ulp

pytestmark = pytest.mark.gpu


class VModel:
    def __init__(self, dims, layers, max_batch=16):
        self.dims = dims
        self.h = torch.zeros(dims["d"], dtype=torch.float32, device=DEV)
        self.hb = torch.zeros(max_batch, dims["d"], dtype=torch.float32, device=DEV)
        self.ws = torch.zeros(q4.workspace_bytes(dims, n_layers=len(layers), max_batch=max_batch),
                              dtype=torch.uint8, device=DEV)
        self.dec = q4.Decoder(dims, layers, self.h, self.ws, EPS, max_batch=max_batch,
                              h_batch=self.hb)

    def run(self, H0, graph, s):
        B = H0.shape[0]
        self.hb[:B].copy_(H0.to(DEV))
        torch.cuda.synchronize()
        (self.dec.verify_graph if graph else self.dec.verify_eager)(B, s)
        s.synchronize()
        return self.hb[:B].cpu().clone()


def columns(dims, config, B):
    return torch.stack([inputs.residual_f32(dims["d"], inputs.seed_of(config, t, 9))
                        for t in range(B)])


@pytest.mark.parametrize("B", [1, 2, 3, 5, 9, 16])
def test_verify_columns_match_oracle(B):
    n = 3
    layers = make_layers(SMALL, 60, n)
    host = to_host(layers)
    m = VModel(SMALL, layers)
    s = torch.cuda.Stream()
    H0 = columns(SMALL, 60, B)
    got = m.run(H0, False, s)
    for b in range(B):
        ref = oracle_run(host, SMALL, H0[b].numpy())
        check_h(got[b].numpy(), ref[-1][0], ref[-1][1], f"verify B={B} column {b}")
    # graph replays (several, with eager work between) equal eager bitwise
    for rep in range(3):
        assert torch.equal(m.run(H0, True, s), got), (B, rep)
        m.run(H0[:1], False, s)


def test_verify_single_column_is_the_decode_step():
    n = 4
    layers = make_layers(TINY, 61, n)
    m = VModel(TINY, layers, max_batch=4)
    s = torch.cuda.Stream()
    h0 = inputs.residual_f32(TINY["d"], inputs.seed_of(61, 0, 9))
    m.h.copy_(h0.to(DEV))
    torch.cuda.synchronize()
    m.dec.step_eager(s)
    s.synchronize()
    assert torch.equal(m.run(h0[None], False, s)[0], m.h.cpu())
    assert torch.equal(m.run(h0[None], True, s)[0], m.h.cpu())


@pytest.mark.parametrize("B", [2, 3])
def test_verify_few_columns_are_decode_steps(B):
    """Two and three columns on shapes whose products all run on the
    vector-ALU batch kernel (columns in the single-token order, the norm in
    the QKV and gate+up prologues exactly as the single-token step computes
    it, the V gather the same binary16 copy): every column equals the
    single-token step of its token bitwise."""
    n = 3
    layers = make_layers(SMALL, 64, n)
    m = VModel(SMALL, layers, max_batch=4)
    s = torch.cuda.Stream()
    H0 = columns(SMALL, 64, B)
    got = m.run(H0, False, s)
    for b in range(B):
        m.h.copy_(H0[b].to(DEV))
        torch.cuda.synchronize()
        m.dec.step_eager(s)
        s.synchronize()
        assert torch.equal(got[b], m.h.cpu()), (B, b)


def test_verify_column_independent_of_batch():
    """Within each product path a column's result does not depend on B or on
    the other columns (bitwise): up to three columns run the vector-ALU batch
    kernel (these shapes fit its LDS stage), four and more the matrix cores."""
    n = 2
    layers = make_layers(SMALL, 62, n)
    m = VModel(SMALL, layers)
    s = torch.cuda.Stream()
    H0 = columns(SMALL, 62, 9)
    full = m.run(H0, False, s)
    for B in (4, 5, 8):
        assert torch.equal(m.run(H0[:B], False, s), full[:B]), B
    perm = torch.tensor([8, 3, 0, 5, 1, 7, 2, 6, 4])
    assert torch.equal(m.run(H0[perm], True, s), full[perm])
    three = m.run(H0[:3], False, s)
    assert torch.equal(m.run(H0[:2], False, s), three[:2])
    perm3 = torch.tensor([2, 0, 1])
    assert torch.equal(m.run(H0[perm3], True, s), three[perm3])


def test_verify_argument_errors():
    layers = make_layers(TINY, 63, 1)
    m = VModel(TINY, layers, max_batch=4)
    s = torch.cuda.Stream()
    for B in (0, 5):
        with pytest.raises(q4.Q4Error, match="INVALID_ARG"):
            m.dec.verify_eager(B, s)
    kv = torch.zeros(q4.kv_cache_elems(SMALL, 1, 64), dtype=torch.int16, device=DEV)
    h = torch.zeros(SMALL["d"], dtype=torch.float32, device=DEV)
    hb = torch.zeros(2, SMALL["d"], dtype=torch.float32, device=DEV)
    ws = torch.zeros(q4.workspace_bytes(SMALL, n_layers=1, max_ctx=64, max_batch=2),
                     dtype=torch.uint8, device=DEV)
    dec = q4.Decoder(SMALL, make_layers(SMALL, 63, 1), h, ws, EPS, kv_cache=kv, max_ctx=64,
                     max_batch=2, h_batch=hb)
    dec.set_context(64, s)
    with pytest.raises(q4.Q4Error, match="INVALID_ARG"):
        dec.verify_eager(2, s)                 # positions 63, 64: past the 64-row cache
    dec.set_context(63, s)
    dec.verify_eager(2, s)                     # positions 62, 63
    s.synchronize()


def test_8b_verify_two_columns_match_oracle():
    """Llama-3-8B shapes, 32 layers, B = 4 graph-captured; columns 0 and 3
    against the oracle."""
    dims = {k: v for k, v in inputs.MODEL_DIMS["8b"].items() if k != "n_layers"}
    layers = make_layers(dims, 2, 32)
    m = VModel(dims, layers, max_batch=9)
    s = torch.cuda.Stream()
    H0 = columns(dims, 64, 4)
    got = m.run(H0, True, s)
    assert torch.equal(m.run(H0, False, s), got)
    host = to_host(layers)
    del layers
    for b in (0, 3):
        ref = oracle_run(host, dims, H0[b].numpy())
        rel = check_h(got[b].numpy(), ref[-1][0], ref[-1][1], f"8b verify column {b}")
        assert rel < 1e-2


# ------------------------------------------------------- attention in the batch
def verify_sections(dims, ws, n_layers, max_ctx, mb, B):
    """qkv (f32 [B][nqkv]) and attention output (binary16 [B][H hd]) of the
    verify step, read from the end of the workspace."""
    a = lambda n: (n + 255) // 256 * 256
    d, H, Hkv, hd, dff = (dims[k] for k in ("d", "H", "Hkv", "hd", "dff"))
    nqkv = (H + 2 * Hkv) * hd
    vb = a(mb * d * 2) + a(mb * nqkv * 4) + a(mb * H * hd * 2) + a(mb * dff * 2)
    total = q4.workspace_bytes(dims, n_layers=n_layers, max_ctx=max_ctx, max_batch=mb)
    o_qkv = total - vb + a(mb * d * 2)
    o_oin = o_qkv + a(mb * nqkv * 4)
    w = ws.cpu()
    qkv = w[o_qkv:o_qkv + B * nqkv * 4].view(torch.float32).numpy().reshape(B, nqkv)
    oin = w[o_oin:o_oin + B * H * hd * 2].view(torch.int16).numpy().view(np.uint16)
    return qkv, oin.reshape(B, H * hd)


def teacher_forced_verify(dims, layers, max_ctx, ctx, B, prefill, H0, what, mb=16):
    """One single-layer decoder per layer over that layer's cache slice, the
    residual columns carried from layer to layer; after each layer the
    attention of every column is checked against the oracle attending, in
    column order, from the GPU's QKV rows (each column sees the rows the
    oracle stored for the columns before it)."""
    Hkv, hd, H = dims["Hkv"], dims["hd"], dims["H"]
    n = len(layers)
    S = Hkv * max_ctx * hd
    kv = torch.from_numpy(prefill.view(np.int16)).to(DEV)
    h = torch.zeros(dims["d"], dtype=torch.float32, device=DEV)
    hb = torch.zeros(mb, dims["d"], dtype=torch.float32, device=DEV)
    hb[:B].copy_(H0.to(DEV))
    s = torch.cuda.Stream()
    worst = 0.0
    for l in range(n):
        kv_l = kv[2 * l * S:2 * (l + 1) * S]
        ws = torch.zeros(q4.workspace_bytes(dims, n_layers=1, max_ctx=max_ctx, max_batch=mb),
                         dtype=torch.uint8, device=DEV)
        dec = q4.Decoder(dims, [layers[l]], h, ws, EPS, kv_cache=kv_l, max_ctx=max_ctx,
                         max_batch=mb, h_batch=hb)
        dec.set_context(ctx, s)
        dec.verify_eager(B, s)
        s.synchronize()
        qkv, oin = verify_sections(dims, ws, 1, max_ctx, mb, B)
        cache = u16(kv_l).reshape(2, Hkv, max_ctx, hd)
        pre = prefill.reshape(n, 2, Hkv, max_ctx, hd)[l]
        kref, vref = np.ascontiguousarray(pre[0]), np.ascontiguousarray(pre[1])
        half = hd // 2
        for b in range(B):
            pos = ctx - 1 + b
            o_ref, mag = oracle.attention(qkv[b].astype(np.float64), dims, pos, kref, vref, BASE)
            v32 = qkv[b, (H + Hkv) * hd:].reshape(Hkv, hd)
            assert np.array_equal(cache[1, :, pos], v32.astype(np.float16).view(np.uint16)), \
                f"{what} layer {l} column {b}: V row"
            k32 = qkv[b, H * hd:(H + Hkv) * hd].reshape(Hkv, hd).astype(np.float64)
            # the rotation's fp32 error: at most 4 * 2^-24 of the pair's norm
            # (derived where the single-token K row is checked)
            norm = np.sqrt(k32[:, :half] ** 2 + k32[:, half:] ** 2)
            norm = np.concatenate([norm, norm], axis=1)
            kw = oracle.f16_to_f64(kref[:, pos])
            kg = oracle.f16_to_f64(cache[0, :, pos])
            kb = f16_ulp(np.maximum(np.abs(kw), np.abs(kg))) + norm * 2.0 ** -22
            assert np.all(np.abs(kg - kw) <= kb), f"{what} layer {l} column {b}: K row"
            got = oracle.f16_to_f64(oin[b])
            bound = 2e-3 * mag + f16_ulp(o_ref) + 1e-6
            err = np.abs(got - o_ref)
            assert np.all(err <= bound), (
                f"{what} layer {l} column {b}: {int((err > bound).sum())} outside, worst "
                f"{float((err / bound).max()):.3g}")
            worst = max(worst, float((err / bound).max()))
        rows = np.ones(max_ctx, bool)
        rows[ctx - 1:ctx - 1 + B] = False
        assert np.array_equal(cache[:, :, rows], pre[:, :, rows]), f"{what} layer {l}: other rows"
        dec.close()
    print(f"{what}: worst attention err/bound {worst:.3g}")
    return hb[:B].cpu().clone(), u16(kv).copy()


@pytest.mark.parametrize("ctx,B", [(1, 2), (60, 9), (120, 16), (192, 9)])
def test_verify_attention_teacher_forced(ctx, B):
    """Draft columns spanning chunk boundaries (positions 59..67, 119..134)
    and the end of a 200-row cache (191..199)."""
    dims = SMALL
    n, max_ctx = 2, 200
    layers = make_layers(dims, 70, n)
    prefill = u16(inputs.act_f16((q4.kv_cache_elems(dims, n, max_ctx),), inputs.seed_of(70, 0, 8)))
    H0 = columns(dims, 70, B)
    teacher_forced_verify(dims, layers, max_ctx, ctx, B, prefill, H0, f"ctx {ctx} B {B}")


@pytest.mark.parametrize("variant,ctx,B", [("qh8_hd128", 120, 16), ("qh8_hd128", 60, 9),
                                           ("qh1_hd64", 120, 16), ("qh4_hd128", 192, 9)])
def test_verify_attention_head_layouts(variant, ctx, B):
    """The draft-batch attention tile for every head layout: 1, 4 and 8
    query heads per group (up to 128 rows of the query matrix, eight row
    tiles), head dims 64 and 128, draft columns across chunk boundaries."""
    dims = VARIANTS[variant]
    n, max_ctx = 1, 200
    layers = make_layers(dims, 72, n)
    prefill = u16(inputs.act_f16((q4.kv_cache_elems(dims, n, max_ctx),), inputs.seed_of(72, 0, 8)))
    H0 = columns(dims, 72, B)
    teacher_forced_verify(dims, layers, max_ctx, ctx, B, prefill, H0, f"{variant} ctx {ctx} B {B}")


def test_verify_attention_paths_agree():
    """With a KV cache: B = 1 equals the single-token step bitwise, graph
    replays equal eager (residual columns and caches), and the resident
    multi-layer decoder equals the chain of single-layer decoders."""
    dims = SMALL
    n, max_ctx, mb, ctx = 3, 200, 16, 100
    layers = make_layers(dims, 71, n)
    prefill = u16(inputs.act_f16((q4.kv_cache_elems(dims, n, max_ctx),), inputs.seed_of(71, 0, 8)))
    kv = torch.empty(q4.kv_cache_elems(dims, n, max_ctx), dtype=torch.int16, device=DEV)
    reset = lambda: (kv.copy_(torch.from_numpy(prefill.view(np.int16)).to(DEV)),
                     torch.cuda.synchronize())
    h = torch.zeros(dims["d"], dtype=torch.float32, device=DEV)
    hb = torch.zeros(mb, dims["d"], dtype=torch.float32, device=DEV)
    ws = torch.zeros(q4.workspace_bytes(dims, n_layers=n, max_ctx=max_ctx, max_batch=mb),
                     dtype=torch.uint8, device=DEV)
    dec = q4.Decoder(dims, layers, h, ws, EPS, kv_cache=kv, max_ctx=max_ctx, max_batch=mb,
                     h_batch=hb)
    s = torch.cuda.Stream()
    H0 = columns(dims, 71, 9)
    # B = 1 against the single-token step
    reset()
    h.copy_(H0[0].to(DEV))
    dec.set_context(ctx, s)
    dec.step_eager(s)
    s.synchronize()
    h_step, c_step = h.cpu().clone(), u16(kv).copy()
    reset()
    hb[:1].copy_(H0[:1].to(DEV))
    dec.set_context(ctx, s)
    dec.verify_eager(1, s)
    s.synchronize()
    assert torch.equal(hb[0].cpu(), h_step) and np.array_equal(u16(kv), c_step)
    # B = 9: eager, graph replays
    reset()
    hb[:9].copy_(H0.to(DEV))
    dec.set_context(ctx, s)
    dec.verify_eager(9, s)
    s.synchronize()
    h_e, c_e = hb[:9].cpu().clone(), u16(kv).copy()
    for rep in range(3):
        reset()
        hb[:9].copy_(H0.to(DEV))
        dec.set_context(ctx, s)
        dec.verify_graph(9, s)
        s.synchronize()
        assert torch.equal(hb[:9].cpu(), h_e), rep
        assert np.array_equal(u16(kv), c_e), rep
    h_tf, c_tf = teacher_forced_verify(dims, layers, max_ctx, ctx, 9, prefill, H0, "chain")
    assert torch.equal(h_tf, h_e) and np.array_equal(c_tf, c_e)


def test_8b_verify_attention_teacher_forced():
    """Llama-3-8B shapes, all 32 layers, 4096-row caches, nine draft
    columns at positions 3990..3998, attention checked at every layer."""
    dims = {k: v for k, v in inputs.MODEL_DIMS["8b"].items() if k != "n_layers"}
    n, max_ctx = 32, 4096
    layers = make_layers(dims, 2, n)
    prefill = u16(inputs.act_f16((q4.kv_cache_elems(dims, n, max_ctx),), inputs.seed_of(2, 0, 8)))
    H0 = columns(dims, 72, 9)
    teacher_forced_verify(dims, layers, max_ctx, 3991, 9, prefill, H0, "8b", mb=9)
