"""Allocation-free decoder layer (q4_decode_layer_noalloc) against the
decoder's own layer entry point (q4_decode_layer with a caller workspace):
the same kernels, so the same bits; both within the product bound of the
free-running oracle.  Two calls in a row on one stream, the second with a
smaller layer, then the larger again (the static array keeps the previous
call's values, which must not leak into the next)."""
import numpy as np
import pytest
import torch

import int4_weight_streaming_q4_amd as q4
import oracle
from int4_weight_streaming_q4_amd import inputs
from helpers import DEV, u16, u8

pytestmark = pytest.mark.gpu

EPS = 1e-5
LARGE = {k: v for k, v in inputs.MODEL_DIMS["8b"].items() if k != "n_layers"}
SMALL = dict(d=64, H=4, Hkv=2, hd=16, dff=96)


def decoder_layer(dims, L, h0):
    """q4_decode_layer on a decoder with a workspace (the existing entry point)."""
    h = torch.zeros(dims["d"], dtype=torch.float32, device=DEV)
    ws = torch.zeros(q4.workspace_bytes(dims, n_layers=1), dtype=torch.uint8, device=DEV)
    dec = q4.Decoder(dims, None, h, ws, EPS, n_layers=1)
    s = torch.cuda.Stream()
    h.copy_(h0.to(DEV))
    torch.cuda.synchronize()
    dec.layer(L, s)
    s.synchronize()
    out = h.cpu().clone()
    dec.close()
    return out


def check_oracle(dims, L, h0, got, what):
    host = {k: (u8(p), u16(sc)) for k, (p, sc) in L.items()}
    h = h0.numpy().astype(np.float64).copy()
    mag = np.zeros_like(h)
    oracle.decode_layer(host, dims, h, mag, EPS)
    g = got.numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), what
    err = np.abs(g - h)
    bound = 2e-3 * mag + 1e-6
    assert np.all(err <= bound), f"{what}: worst err/bound {float((err / bound).max()):.3g}"


def test_noalloc_layer_equals_decoder_layer():
    cases = []
    for name, dims, cfg in (("8B layer", LARGE, 61), ("small layer", SMALL, 62)):
        L = inputs.layer_weights(dims, cfg, 0, device=DEV)
        h0 = inputs.residual_f32(dims["d"], inputs.seed_of(cfg, 0, 9))
        cases.append((name, dims, L, h0, decoder_layer(dims, L, h0)))
    s = torch.cuda.Stream()
    # large, then small, then large again, back to back on one stream
    order = [0, 1, 0]
    hs = [torch.empty(cases[i][1]["d"], dtype=torch.float32, device=DEV) for i in order]
    for i, h in zip(order, hs):
        h.copy_(cases[i][3].to(DEV))
    torch.cuda.synchronize()
    for i, h in zip(order, hs):
        name, dims, L, h0, want = cases[i]
        q4.decode_layer_noalloc(L, dims, h, EPS, s)
    s.synchronize()
    for i, h in zip(order, hs):
        name, dims, L, h0, want = cases[i]
        got = h.cpu()
        assert torch.equal(got, want), name
        check_oracle(dims, L, h0, got, name)
