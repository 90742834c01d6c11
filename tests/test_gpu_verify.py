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

import int4_weight_streaming_q4_amd as q4
from int4_weight_streaming_q4_amd import inputs
from helpers import DEV
from test_gpu_decode import SMALL, TINY, EPS, check_h, make_layers, oracle_run, to_host

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


def test_verify_column_independent_of_batch():
    n = 2
    layers = make_layers(SMALL, 62, n)
    m = VModel(SMALL, layers)
    s = torch.cuda.Stream()
    H0 = columns(SMALL, 62, 9)
    full = m.run(H0, False, s)
    for B in (2, 4, 8):
        assert torch.equal(m.run(H0[:B], False, s), full[:B]), B
    perm = torch.tensor([8, 3, 0, 5, 1, 7, 2, 6, 4])
    assert torch.equal(m.run(H0[perm], True, s), full[perm])


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
    with pytest.raises(q4.Q4Error, match="UNSUPPORTED"):
        dec.verify_eager(2, s)


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
