"""GPU parity of q4_quantize against the oracle: codes and scales bit-exact
(an integer decided by floating point, taken in the same binary32 division
on both sides).  Inputs: seeded N(0,1) weights times a per-row magnitude
(binary32 and binary16), groups built to hit the rule's edges, and, at the
Llama-3-8B gate+up shape, weights on the quantization grid, which must come
back as the codes and scales they were built from."""
import numpy as np
import pytest
import torch

import oracle
import int4_weight_streaming_q4_amd as q4
from int4_weight_streaming_q4_amd import inputs
from helpers import DEV, u16, u8

pytestmark = pytest.mark.gpu


def gpu_quantize(w_dev):
    N, K = w_dev.shape
    packed = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(N, K // 32, dtype=torch.int16, device=DEV)
    q4.q4_quantize(w_dev, packed, scales)
    torch.cuda.synchronize()
    return u8(packed), u16(scales)


def oracle_quantize(w_host):
    codes, scales = oracle.quantize(w_host)
    return oracle.pack(codes), scales


def random_weights(N, K, seed):
    g = torch.Generator().manual_seed(seed)
    mag = torch.rand(N, 1, generator=g) * 3.0 + 1e-3
    return (torch.randn(N, K, generator=g) * mag).float()


@pytest.mark.parametrize("N,K", [(1, 32), (37, 416), (128, 4096), (5, 14336)])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_quantize_matches_oracle(N, K, dtype):
    w = random_weights(N, K, 100 + N + K)
    if dtype == "f16":
        w16 = w.half()
        got = gpu_quantize(w16.to(DEV))
        want = oracle_quantize(w16.view(torch.int16).numpy().view(np.uint16))
    else:
        got = gpu_quantize(w.to(DEV))
        want = oracle_quantize(w.numpy())
    assert np.array_equal(got[1], want[1]), "scales"
    assert np.array_equal(got[0], want[0]), "codes"


def test_quantize_edge_groups():
    """Ties (w / s = k + 0.5), clips at +8 s, zero and tiny groups, a
    subnormal scale, negative zeros, the largest binary16 magnitudes, and a
    quotient that is exactly a tie in binary32 but not via a reciprocal."""
    K = 32
    rows = []
    r = np.zeros(K, np.float32); r[:12] = [8, -8, .5, 1.5, 2.5, -.5, -1.5, -2.5, 3.49, 6.75, -7.6, 7.5]
    rows.append(r)
    rows.append(np.zeros(K, np.float32))                          # zero group
    rows.append(np.full(K, 2.0 ** -28, np.float32))               # scale rounds to 0
    r = np.zeros(K, np.float32); r[0] = -0.0; r[1] = 2.0 ** -20; r[2] = -(2.0 ** -21)
    rows.append(r)                                                # subnormal scale
    r = np.linspace(-65504.0, 65504.0, K).astype(np.float32)
    rows.append(r)                                                # largest binary16 values
    s = np.float32(np.float16(1.612))
    r = np.zeros(K, np.float32); r[0] = 8 * s; r[1] = np.float32(float.fromhex("0x1.6928p+2"))
    rows.append(r)
    rng = np.random.default_rng(7)
    for _ in range(10):                                           # many exact ties
        s = np.float32(np.float16(rng.uniform(0.01, 4)))
        k = rng.integers(-8, 8, K).astype(np.float32)
        r = ((k + np.float32(0.5)) * s).astype(np.float32)
        r[0] = 8 * s
        rows.append(r)
    w = np.stack(rows).astype(np.float32)
    got = gpu_quantize(torch.from_numpy(w).to(DEV))
    want = oracle_quantize(w)
    assert np.array_equal(got[1], want[1])
    assert np.array_equal(got[0], want[0])
    codes = oracle.unpack(got[0])
    assert codes[0, 0] == 15 and codes[0, 7] == 6 and codes[1].tolist() == [8] * K
    assert got[1][1, 0] == 0 and got[1][2, 0] == 0 and codes[5, 1] == 12


def test_quantize_gate_up_shape_recovers_grid_weights():
    """At the 8B gate+up shape (28672 x 4096), weights built as s * (c - 8)
    from seeded codes and scales, with code 0 in every group (so max|w| =
    8 s), quantize back to exactly those bytes, as binary32 and as
    binary16.  Sampled rows of random weights also match the oracle."""
    N, K = 28672, 4096
    packed0 = inputs.random_bytes(N, K, inputs.seed_of(3, 40, 0), device=DEV)
    packed0.view(N, K // 32, 16)[:, :, 0] &= 0xF0                 # code 0 at k = 32 g
    # scales with 4 significant bits (2^-e * (1 + j/8)), so every s * (c - 8)
    # is exact in binary16 as well as binary32
    g = torch.Generator(device=DEV).manual_seed(inputs.seed_of(3, 40, 1))
    e = torch.randint(4, 11, (N, K // 32), generator=g, device=DEV).float()
    j = torch.randint(0, 8, (N, K // 32), generator=g, device=DEV).float()
    scales0 = (torch.pow(2.0, -e) * (1.0 + j / 8.0)).half().view(torch.int16)
    lo = (packed0 & 0x0F).to(torch.int16)
    hi = (packed0 >> 4).to(torch.int16)
    codes = torch.stack([lo, hi], dim=2).reshape(N, K)
    s = scales0.view(torch.float16).float().repeat_interleave(32, dim=1)
    w32 = (codes.float() - 8.0) * s                               # exact in binary32
    for w in (w32, w32.half()):
        p, sc = gpu_quantize(w)
        assert np.array_equal(sc, u16(scales0))
        assert np.array_equal(p, u8(packed0))
    rows = np.random.default_rng(3).choice(N, 48, replace=False)
    wr = np.random.default_rng(4).standard_normal((48, K)).astype(np.float32)
    w_dev = torch.zeros(N, K, dtype=torch.float32, device=DEV)
    w_dev[torch.from_numpy(rows).to(DEV)] = torch.from_numpy(wr).to(DEV)
    p, sc = gpu_quantize(w_dev)
    wp, ws = oracle_quantize(wr)
    assert np.array_equal(p[rows], wp) and np.array_equal(sc[rows], ws)
