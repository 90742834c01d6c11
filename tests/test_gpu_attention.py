"""GPU parity of decode attention over binary16 KV caches against the oracle.

Attention of a step reads the caches written by earlier tokens; those rows
are inputs here, prefilled with seeded binary16 N(0,1) values (the activation
generator), so any position can be tested directly.  Each check is teacher
forced: after the QKV product and attention of a layer, the oracle attends
from the GPU's own fp32 QKV output over the same prefilled rows, in fp64.

* the new cache row: V exactly the binary16 rounding of the GPU's V rows, the
  rotated K within one binary16 ulp of the oracle's plus 2^-22 times the
  norm of the rotated pair (three fp32 roundings: the rotation runs in
  fp32 on the GPU, in fp64 in
  the oracle);
* the attention output: |o - o_ref| <= 2e-3 * sum_j p_j |v_j| + ulp16(o_ref)
  + 1e-6 per element (the product bound applied to the weighted value sum,
  plus the binary16 rounding of the output);
* every other cache row unchanged.
Eager steps, graph replays, layer-by-layer steps and streamed tokens over the
same caches agree bitwise.
"""
import numpy as np
import pytest
import torch

import oracle
import int4_weight_streaming_q4_amd as q4
from int4_weight_streaming_q4_amd import inputs
from helpers import DEV, u16, u8
from test_gpu_wstream import blobs_for

pytestmark = pytest.mark.gpu

EPS = 1e-5
BASE = 500000.0

# query heads per key/value head 2, 8, 1, 4; head dims 64 and 128
VARIANTS = {
    "qh2_hd64": dict(d=256, H=4, Hkv=2, hd=64, dff=384),
    "qh8_hd128": dict(d=256, H=8, Hkv=1, hd=128, dff=256),
    "qh1_hd64": dict(d=256, H=4, Hkv=4, hd=64, dff=320),
    "qh4_hd128": dict(d=512, H=8, Hkv=2, hd=128, dff=384),
}


def f16_ulp(v):
    a = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(a)) - 10)


class KVModel:
    """Decoder with a KV cache plus the device buffers it retains."""

    def __init__(self, dims, layers, n_layers, max_ctx, resident=True, prefill_seed=None):
        self.dims, self.n, self.max_ctx = dims, n_layers, max_ctx
        self.h = torch.zeros(dims["d"], dtype=torch.float32, device=DEV)
        n_el = q4.kv_cache_elems(dims, n_layers, max_ctx)
        if prefill_seed is None:
            self.prefill = np.zeros(n_el, np.uint16)
        else:
            self.prefill = u16(inputs.act_f16((n_el,), prefill_seed))
        self.kv = torch.empty(n_el, dtype=torch.int16, device=DEV)
        self.reset_cache()
        self.ws = torch.zeros(q4.workspace_bytes(dims, n_layers=n_layers, max_ctx=max_ctx),
                              dtype=torch.uint8, device=DEV)
        self.dec = q4.Decoder(dims, layers if resident else None, self.h, self.ws, EPS,
                              n_layers=n_layers, kv_cache=self.kv, max_ctx=max_ctx,
                              rope_base=BASE)

    def reset_cache(self):
        self.kv.copy_(torch.from_numpy(self.prefill.view(np.int16)).to(DEV))
        torch.cuda.synchronize()

    def set_h(self, h0):
        self.h.copy_(torch.as_tensor(h0, dtype=torch.float32, device=DEV))
        torch.cuda.synchronize()

    def shape5(self):
        d = self.dims
        return (self.n, 2, d["Hkv"], self.max_ctx, d["hd"])

    def host_slices(self, l):
        """Copies of the prefilled K and V caches of layer l."""
        c = self.prefill.reshape(self.shape5())
        return np.ascontiguousarray(c[l, 0]), np.ascontiguousarray(c[l, 1])

    def gpu_rows(self, l, pos):
        """The GPU's K and V cache rows `pos` of layer l, [Hkv][hd] each."""
        c = self.kv.view(self.shape5())
        return u16(c[l, 0, :, pos, :]), u16(c[l, 1, :, pos, :])

    def cache(self):
        return u16(self.kv).reshape(self.shape5())

    def sections(self):
        d = self.dims
        a = lambda n: (n + 255) // 256 * 256
        o1 = a(max(d["d"], d["dff"]) * 2)
        nqkv = (d["H"] + 2 * d["Hkv"]) * d["hd"]
        o2 = o1 + a(nqkv * 4)
        ws = self.ws.cpu()
        qkv = ws[o1:o1 + nqkv * 4].view(torch.float32).numpy()
        oin = ws[o2:o2 + d["H"] * d["hd"] * 2].view(torch.int16).numpy().view(np.uint16)
        return qkv, oin


def check_attention(m, l, pos, what):
    """Teacher-forced check of layer l's attention at position pos, run
    right after the layer's QKV product and attention."""
    d = m.dims
    qkv, oin = m.sections()
    kref, vref = m.host_slices(l)
    o_ref, mag = oracle.attention(qkv.astype(np.float64), d, pos, kref, vref, BASE)
    kg, vg = m.gpu_rows(l, pos)
    # V row: the binary16 rounding of the GPU's fp32 V
    v32 = qkv[(d["H"] + d["Hkv"]) * d["hd"]:].reshape(d["Hkv"], d["hd"])
    assert np.array_equal(vg, v32.astype(np.float16).view(np.uint16)), f"{what}: V row"
    # K row.  Both sides rotate the same fp32 pair (a, b) by the same angle;
    # the oracle in fp64, the GPU in fp32 from a table whose cos and sin
    # were taken in fp64 and rounded to fp32 once.  With u = 2^-24, the GPU
    # value r of a c - b s (or a s + b c) carries at most three roundings
    # of relative size u -- the table entry, the product, the difference
    # (a fused multiply-add only removes one) -- each scaled by a term of
    # the sum, so |r - R| <= 3u (|a||c| + |b||s|) (1 + 2u)
    # <= 3u sqrt(a^2 + b^2) (1 + 2u) (Cauchy-Schwarz, c^2 + s^2 = 1); the
    # fp64 angles and sums of both sides differ by less than 2^-40 of the
    # same norm.  4u sqrt(a^2 + b^2) covers all of it.  Where the rotation
    # cancels this exceeds a binary16 ulp of the result; then each side
    # rounds to binary16, half an ulp each.
    kw = oracle.f16_to_f64(kref[:, pos, :])
    kgot = oracle.f16_to_f64(kg)
    k32 = qkv[d["H"] * d["hd"]:(d["H"] + d["Hkv"]) * d["hd"]].reshape(d["Hkv"], d["hd"])
    half = d["hd"] // 2
    k64 = k32.astype(np.float64)
    norm = np.sqrt(k64[:, :half] ** 2 + k64[:, half:] ** 2)
    norm = np.concatenate([norm, norm], axis=1)
    kbound = f16_ulp(np.maximum(np.abs(kw), np.abs(kgot))) + norm * 2.0 ** -22
    assert np.all(np.abs(kgot - kw) <= kbound), f"{what}: rotated K row"
    got = oracle.f16_to_f64(oin)
    bound = 2e-3 * mag + f16_ulp(o_ref) + 1e-6
    err = np.abs(got - o_ref)
    assert np.all(np.isfinite(got)), what
    assert np.all(err <= bound), (
        f"{what}: {int((err > bound).sum())} outputs outside; worst err/bound "
        f"{float((err / bound).max()):.3g}")
    return float((err / bound).max())


def check_other_rows(m, pos):
    """Only row pos of every cache changed."""
    got = m.cache().copy()
    want = m.prefill.reshape(m.shape5()).copy()
    got[:, :, :, pos, :] = 0
    want[:, :, :, pos, :] = 0
    assert np.array_equal(got, want), "a cache row other than the current position changed"


def teacher_forced_token(m, layers, pos, h0, s, what):
    m.reset_cache()
    m.set_h(h0)
    m.dec.set_context(pos + 1, s)
    worst = 0.0
    for l in range(m.n):
        m.dec.layer_part(layers[l], 0, s)
        s.synchronize()
        worst = max(worst, check_attention(m, l, pos, f"{what} layer {l}"))
        for which in (1, 2, 3):
            m.dec.layer_part(layers[l], which, s)
    s.synchronize()
    check_other_rows(m, pos)
    print(f"{what}: worst attention err/bound {worst:.3g}")
    return m.h.cpu().clone(), m.cache().copy()


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_attention_positions_match_oracle(variant):
    """Two layers driven product by product; positions at the first row, on
    both sides of chunk boundaries and the last row of a cache whose length
    (200) is not a multiple of the 64-position chunk."""
    dims = VARIANTS[variant]
    n, max_ctx = 2, 200
    layers = [inputs.layer_weights(dims, 30, l, device=DEV) for l in range(n)]
    m = KVModel(dims, layers, n, max_ctx, resident=False,
                prefill_seed=inputs.seed_of(30, 0, 8))
    s = torch.cuda.Stream()
    for pos in (0, 1, 63, 64, 100, 127, 128, 199):
        h0 = inputs.residual_f32(dims["d"], inputs.seed_of(30, pos, 9))
        teacher_forced_token(m, layers, pos, h0, s, f"{variant} pos {pos}")


def test_attention_beyond_one_merge_round():
    """Contexts past 4096 positions (eager steps): more than 64 chunk
    partials, so the merge runs a second round of chunks with a running
    maximum; positions on both sides of the 64th chunk boundary and the
    last row of a 4200-row cache."""
    dims = VARIANTS["qh4_hd128"]
    n, max_ctx = 2, 4200
    layers = [inputs.layer_weights(dims, 33, l, device=DEV) for l in range(n)]
    m = KVModel(dims, layers, n, max_ctx, resident=False,
                prefill_seed=inputs.seed_of(33, 0, 8))
    s = torch.cuda.Stream()
    for pos in (4095, 4096, 4159, 4160, 4199):
        h0 = inputs.residual_f32(dims["d"], inputs.seed_of(33, pos, 9))
        teacher_forced_token(m, layers, pos, h0, s, f"qh4_hd128 pos {pos}")


def test_attention_wide_model_rows():
    """A model width of 8192 (Llama-3-70B's: 64 query heads, 8 key/value
    heads): the QKV product runs the phased row kernel, whose epilogue
    rotates the query and key rows and stores the token's cache rows."""
    dims = dict(d=8192, H=64, Hkv=8, hd=128, dff=256)
    n, max_ctx = 1, 300
    layers = [inputs.layer_weights(dims, 34, l, device=DEV) for l in range(n)]
    m = KVModel(dims, layers, n, max_ctx, resident=False,
                prefill_seed=inputs.seed_of(34, 0, 8))
    s = torch.cuda.Stream()
    for pos in (0, 65, 299):
        h0 = inputs.residual_f32(dims["d"], inputs.seed_of(34, pos, 9))
        teacher_forced_token(m, layers, pos, h0, s, f"d8192 pos {pos}")


def test_attention_context_one_is_the_one_token_step():
    """At context length 1 the softmax has one term: the attention output is
    the binary16 V of the group, and the step equals the decoder without a
    cache bitwise."""
    dims = VARIANTS["qh2_hd64"]
    n = 3
    layers = [inputs.layer_weights(dims, 31, l, device=DEV) for l in range(n)]
    h0 = inputs.residual_f32(dims["d"], inputs.seed_of(31, 0, 9))
    s = torch.cuda.Stream()
    h = torch.zeros(dims["d"], dtype=torch.float32, device=DEV)
    ws = torch.zeros(q4.workspace_bytes(dims, n_layers=n), dtype=torch.uint8, device=DEV)
    plain = q4.Decoder(dims, layers, h, ws, EPS)
    h.copy_(h0.to(DEV))
    torch.cuda.synchronize()
    plain.step_eager(s)
    s.synchronize()
    h_plain = h.cpu().clone()
    m = KVModel(dims, layers, n, 64, prefill_seed=inputs.seed_of(31, 0, 8))
    m.set_h(h0)
    m.dec.set_context(1, s)
    m.dec.step_eager(s)
    s.synchronize()
    assert torch.equal(m.h.cpu(), h_plain)
    m.reset_cache()
    m.set_h(h0)
    m.dec.step_graph(1, s)
    s.synchronize()
    assert torch.equal(m.h.cpu(), h_plain)


def test_attention_step_paths_agree_bitwise():
    """Eager step, graph replays (one graph serves every context length of
    its bucket), layer-by-layer steps and streamed tokens: same residual and
    same caches bitwise, the streamed token within rel. L2 1e-2 of the
    free-running oracle; argument errors reported."""
    dims = VARIANTS["qh2_hd64"]
    n, max_ctx = 3, 200
    layers = [inputs.layer_weights(dims, 32, l, device=DEV) for l in range(n)]
    host = [{k: (u8(p), u16(sc)) for k, (p, sc) in L.items()} for L in layers]
    m = KVModel(dims, layers, n, max_ctx, prefill_seed=inputs.seed_of(32, 0, 8))
    lw = KVModel(dims, None, n, max_ctx, resident=False, prefill_seed=inputs.seed_of(32, 0, 8))
    st = KVModel(dims, None, n, max_ctx, resident=False, prefill_seed=inputs.seed_of(32, 0, 8))
    blobs, total = blobs_for(dims, layers)
    slots = [torch.empty(total, dtype=torch.uint8, device=DEV) for _ in range(2)]
    copy = torch.cuda.Stream()
    wstream = q4.WeightStream(blobs, slots, copy)
    s = torch.cuda.Stream()
    for ctx in (1, 64, 65, 200, 130):
        h0 = inputs.residual_f32(dims["d"], inputs.seed_of(32, ctx, 9))
        m.reset_cache()
        m.set_h(h0)
        m.dec.set_context(ctx, s)
        m.dec.step_eager(s)
        s.synchronize()
        h_e, c_e = m.h.cpu().clone(), m.cache().copy()
        for rep in range(2):
            m.reset_cache()
            m.set_h(h0)
            m.dec.step_graph(ctx, s)
            s.synchronize()
            assert torch.equal(m.h.cpu(), h_e), (ctx, rep)
            assert np.array_equal(m.cache(), c_e), (ctx, rep)
        lw.reset_cache()
        lw.set_h(h0)
        lw.dec.set_context(ctx, s)
        for l in range(n):
            lw.dec.layer(layers[l], s)
        s.synchronize()
        assert torch.equal(lw.h.cpu(), h_e), ctx
        assert np.array_equal(lw.cache(), c_e), ctx
        st.reset_cache()
        c0 = st.cache().copy()
        st.set_h(h0)
        st.dec.set_context(ctx, s)
        st.dec.token_streamed(wstream, s)
        s.synchronize()
        assert torch.equal(st.h.cpu(), h_e), ctx
        assert np.array_equal(st.cache(), c_e), ctx
        # the streamed token against the free-running oracle from the same caches
        h = h0.numpy().astype(np.float64)
        for l in range(n):
            kc, vc = c0[l, 0].copy(), c0[l, 1].copy()
            oracle.decode_layer_attn(host[l], dims, h, ctx - 1, kc, vc, None, EPS, BASE)
            got_k = oracle.f16_to_f64(st.cache()[l, 0, :, ctx - 1])
            want_k = oracle.f16_to_f64(kc[:, ctx - 1])
            assert np.linalg.norm(got_k - want_k) <= 1e-2 * np.linalg.norm(want_k), (ctx, l)
        got = st.h.cpu().numpy().astype(np.float64)
        rel = float(np.linalg.norm(got - h) / np.linalg.norm(h))
        assert rel < 1e-2, (ctx, rel)
    copy.synchronize()
    with pytest.raises(q4.Q4Error, match="INVALID_ARG"):
        m.dec.step_graph(max_ctx + 1, s)
    for bad in (0, max_ctx + 1):
        with pytest.raises(q4.Q4Error, match="INVALID_ARG"):
            m.dec.set_context(bad, s)
    for mode in (1, 2, 3):
        with pytest.raises(q4.Q4Error, match="UNSUPPORTED"):
            m.dec.set_persistent(mode)
    prof = m.dec.step_profiled(s)
    assert len(prof) == 5 * n and all(x > 0 for x in prof)
    wstream.close()


def test_attention_token_loop_tracks_oracle():
    """70 tokens written into empty caches (crossing a chunk boundary),
    graph-captured, against the oracle running free with its own caches:
    residual per token and the cache rows written within rel L2 1e-2 of the
    oracle's, no row past the context written."""
    dims = VARIANTS["qh2_hd64"]
    n, max_ctx, T = 2, 128, 70
    layers = [inputs.layer_weights(dims, 33, l, device=DEV) for l in range(n)]
    host = [{k: (u8(p), u16(sc)) for k, (p, sc) in L.items()} for L in layers]
    m = KVModel(dims, layers, n, max_ctx)
    caches = [oracle.kv_cache(dims, max_ctx) for _ in range(n)]
    s = torch.cuda.Stream()
    worst = 0.0
    for t in range(T):
        h0 = inputs.residual_f32(dims["d"], inputs.seed_of(33, t, 9))
        m.set_h(h0)
        m.dec.step_graph(t + 1, s)
        s.synchronize()
        h = h0.numpy().astype(np.float64)
        for l in range(n):
            oracle.decode_layer_attn(host[l], dims, h, t, caches[l][0], caches[l][1], None,
                                     EPS, BASE)
        got = m.h.cpu().numpy().astype(np.float64)
        rel = float(np.linalg.norm(got - h) / np.linalg.norm(h))
        worst = max(worst, rel)
        assert rel < 1e-2, (t, rel)
    c = m.cache()
    for l in range(n):
        for kv in (0, 1):
            want = oracle.f16_to_f64(caches[l][kv][:, :T])
            got = oracle.f16_to_f64(c[l, kv, :, :T])
            rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
            assert rel < 1e-2, (l, kv, rel)
        assert not c[l, :, :, T:].any(), "rows past the context were written"
    print(f"token loop: worst rel L2 {worst:.3g}")


def test_8b_attention_teacher_forced_all_layers():
    """Llama-3-8B shapes, 32 resident layers, caches of 4096 rows: attention
    of every layer checked at positions 4095 (a full 4096 bucket) and 1000;
    the graph step then gives the same residual and caches bitwise."""
    dims = {k: v for k, v in inputs.MODEL_DIMS["8b"].items() if k != "n_layers"}
    n, max_ctx = 32, 4096
    layers = [inputs.layer_weights(dims, 2, l, device=DEV) for l in range(n)]
    m = KVModel(dims, layers, n, max_ctx, prefill_seed=inputs.seed_of(2, 0, 8))
    s = torch.cuda.Stream()
    for pos in (4095, 1000):
        h0 = inputs.residual_f32(dims["d"], inputs.seed_of(2, pos, 9))
        h_parts, c_parts = teacher_forced_token(m, layers, pos, h0, s, f"8b pos {pos}")
        m.reset_cache()
        m.set_h(h0)
        m.dec.step_graph(pos + 1, s)
        s.synchronize()
        assert torch.equal(m.h.cpu(), h_parts), pos
        assert np.array_equal(m.cache(), c_parts), pos
