"""Pins that tie the CPU oracle to something other than itself.

Each test checks the oracle against a library routine, a closed form, an
invariant or a brute-force path written independently here, chosen so that a
dropped term, a wrong sign or index, or a transposed operand fails at least
one of them.  No GPU is needed.
"""
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f16_bits(v):
    return np.asarray(v, np.float64).astype(np.float16).view(np.uint16)


def _rand_mat(rng, N, K, scale_kind="random"):
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    if scale_kind == "random":
        s = (np.abs(rng.standard_normal((N, K // 32))) * 0.02).astype(np.float16)
    elif scale_kind == "int":
        s = rng.integers(1, 4, size=(N, K // 32)).astype(np.float16)
    else:
        raise ValueError(scale_kind)
    return codes, s


# ------------------------------------------------------------- binary16
def test_f16_decode_exhaustive():
    """All 65,536 bit patterns decode exactly as numpy's float16."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero and the subnormal/normal boundary, explicitly
    assert np.signbit(oracle.f16_to_f64(np.array([0x8000], np.uint16))[0])
    assert oracle.f16_to_f64(np.array([0x0001], np.uint16))[0] == 2.0 ** -24
    assert oracle.f16_to_f64(np.array([0x0400], np.uint16))[0] == 2.0 ** -14


def test_f16_round_nearest_even():
    """f64 -> f16 agrees with numpy's correctly rounded conversion on exact
    values, on every rounding midpoint and next to it, and at overflow."""
    bits = np.arange(0x7C00, dtype=np.uint16)  # all finite non-negative
    vals = bits.view(np.float16).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2.0  # exact midpoints between neighbours
    cases = [vals, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf)]
    rng = np.random.default_rng(1)
    cases.append(rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 5, 200000))
    cases.append(np.array([65504.0, 65519.99, 65520.0, 70000.0, 1e300, 2.0 ** -25,
                           2.0 ** -25 * 1.0000001, 3 * 2.0 ** -25, 2.0 ** -26]))
    for c in cases:
        for v in (c, -c):
            ours = oracle.f64_to_f16(v)
            with np.errstate(over="ignore"):
                ref = v.astype(np.float16).view(np.uint16)
            assert np.array_equal(ours, ref), v[ours != ref][:5]
    assert oracle.f64_to_f16(np.array([np.nan]))[0] & 0x7C00 == 0x7C00


# ------------------------------------------------------------- packing
def test_pack_unpack_all_bytes_and_pairs():
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    c = oracle.unpack(b)
    assert np.array_equal(c[0, 0::2], np.arange(256) & 0xF)
    assert np.array_equal(c[0, 1::2], np.arange(256) >> 4)
    assert np.array_equal(oracle.pack(c), b)
    lo, hi = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    pairs = np.stack([lo.ravel(), hi.ravel()], axis=1).reshape(1, 512).astype(np.uint8)
    packed = oracle.pack(pairs)
    assert np.array_equal(packed[0], (lo.ravel() | (hi.ravel() << 4)).astype(np.uint8))


def test_pack_masks_high_bits():
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 256, size=(7, 64), dtype=np.uint8)
    assert np.array_equal(oracle.pack(codes), oracle.pack(codes & 0xF))
    assert np.array_equal(oracle.unpack(oracle.pack(codes)), codes & 0xF)


# ------------------------------------------------------------- products
def _dense_reference(codes, s_f16, x):
    """Independent path: build W in numpy from the codes and float16 scales."""
    s = s_f16.astype(np.float64)
    W = np.repeat(s, 32, axis=1) * (codes.astype(np.float64) - 8.0)
    return W @ x, W


def test_brute_force_8x64_exact_integers():
    rng = np.random.default_rng(3)
    codes, s = _rand_mat(rng, 8, 64, "int")
    x = rng.integers(-4, 5, size=64).astype(np.float16)
    y, m = oracle.gemv(oracle.pack(codes), s.view(np.uint16), x.view(np.uint16))
    yr, W = _dense_reference(codes, s, x.astype(np.float64))
    assert np.array_equal(y, yr)
    assert np.array_equal(m, np.abs(W * x.astype(np.float64)).sum(axis=1))
    assert np.array_equal(oracle.dequant(oracle.pack(codes), s.view(np.uint16)), W)


def test_brute_force_8x64_random():
    rng = np.random.default_rng(4)
    codes, s = _rand_mat(rng, 8, 64)
    x = rng.standard_normal(64).astype(np.float16)
    y, _ = oracle.gemv(oracle.pack(codes), s.view(np.uint16), x.view(np.uint16))
    yr, _ = _dense_reference(codes, s, x.astype(np.float64))
    np.testing.assert_allclose(y, yr, rtol=1e-12, atol=1e-15)


def test_allones_closed_form_and_hand_case():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "allones_hand_case.txt"))
            if l.strip() and not l.startswith("#")]
    codes = (np.arange(32) % 16).astype(np.uint8).reshape(1, 32)
    ones = _f16_bits(np.ones(32))
    for sc, expect in rows:
        s = _f16_bits([[float(sc)]])
        y, _ = oracle.gemv(oracle.pack(codes), s, ones)
        assert y[0] == float(expect)
    # closed form on a random matrix: y_n = sum_g s_ng * (sum_{k in g} c_nk - 256)
    rng = np.random.default_rng(5)
    codes, s = _rand_mat(rng, 16, 256)
    y, _ = oracle.gemv(oracle.pack(codes), s.view(np.uint16), _f16_bits(np.ones(256)))
    gsum = codes.reshape(16, 8, 32).astype(np.int64).sum(axis=2) - 256
    closed = (s.astype(np.float64) * gsum).sum(axis=1)
    np.testing.assert_allclose(y, closed, rtol=1e-15, atol=0)


def test_zero_point_gives_exact_zero():
    rng = np.random.default_rng(6)
    codes = np.full((5, 128), 8, np.uint8)
    s = (np.abs(rng.standard_normal((5, 4))) + 0.1).astype(np.float16)
    x = rng.standard_normal(128).astype(np.float16)
    y, m = oracle.gemv(oracle.pack(codes), s.view(np.uint16), x.view(np.uint16))
    assert np.all(y == 0.0) and np.all(m == 0.0)


def test_impulse_picks_one_weight():
    rng = np.random.default_rng(7)
    codes, s = _rand_mat(rng, 6, 96)
    packed = oracle.pack(codes)
    for k in (0, 1, 31, 32, 63, 95):
        x = np.zeros(96)
        x[k] = 1.0
        y, _ = oracle.gemv(packed, s.view(np.uint16), _f16_bits(x))
        expect = s[:, k // 32].astype(np.float64) * (codes[:, k].astype(np.float64) - 8)
        assert np.array_equal(y, expect)


def test_linearity_small_integers():
    rng = np.random.default_rng(8)
    codes, s = _rand_mat(rng, 12, 512)
    packed, sb = oracle.pack(codes), s.view(np.uint16)
    x1 = rng.integers(-4, 5, 512).astype(np.float64)
    x2 = rng.integers(-4, 5, 512).astype(np.float64)
    y1, _ = oracle.gemv(packed, sb, _f16_bits(x1))
    y2, _ = oracle.gemv(packed, sb, _f16_bits(x2))
    y12, _ = oracle.gemv(packed, sb, _f16_bits(x1 + x2))
    y1d, _ = oracle.gemv(packed, sb, _f16_bits(2 * x1))
    assert np.array_equal(y12, y1 + y2)
    assert np.array_equal(y1d, 2 * y1)
    yneg, _ = oracle.gemv(packed, sb, _f16_bits(-x1))
    assert np.array_equal(yneg, -y1)


def test_gemm_is_stacked_gemv_and_rows_subset():
    rng = np.random.default_rng(9)
    codes, s = _rand_mat(rng, 40, 160)
    packed, sb = oracle.pack(codes), s.view(np.uint16)
    X = rng.standard_normal((5, 160)).astype(np.float16)
    Y, M = oracle.gemm(packed, sb, X.view(np.uint16))
    for b in range(5):
        y, m = oracle.gemv(packed, sb, X[b].view(np.uint16))
        assert np.array_equal(Y[b], y) and np.array_equal(M[b], m)
    rows = np.array([39, 0, 17, 17], np.int64)
    yr, mr = oracle.gemv_rows(packed, sb, X[2].view(np.uint16), rows)
    assert np.array_equal(yr, Y[2][rows]) and np.array_equal(mr, M[2][rows])
    # the row/column roles: a transposed product would not match the dense one
    yd, _ = _dense_reference(codes, s, X[3].astype(np.float64))
    np.testing.assert_allclose(Y[3], yd, rtol=1e-12, atol=1e-15)


def test_subnormal_scales_are_honoured():
    codes = np.full((1, 32), 9, np.uint8)  # w = s
    s = np.array([[0x0001]], np.uint16)  # 2^-24
    y, _ = oracle.gemv(oracle.pack(codes), s, _f16_bits(np.ones(32)))
    assert y[0] == 32 * 2.0 ** -24


# ------------------------------------------------------------- glue
def test_rmsnorm_closed_forms():
    for c in (2.0, -0.375, 1e-3):
        a = oracle.rmsnorm_f16(np.full(64, c))
        expect = _f16_bits([c / np.sqrt(c * c + 1e-5)])[0]
        assert np.all(a == expect)
    a = oracle.rmsnorm_f16(np.array([1.0, -1.0] * 16))
    assert np.array_equal(a, _f16_bits([1.0, -1.0] * 16))
    rng = np.random.default_rng(10)
    h = rng.standard_normal(128)
    # with eps = 0 the norm is exactly invariant to power-of-two scaling
    assert np.array_equal(oracle.rmsnorm_f16(h, eps=0.0),
                          oracle.rmsnorm_f16(h * 8.0, eps=0.0))
    assert np.array_equal(oracle.rmsnorm_f16(-h, eps=0.0),
                          oracle.rmsnorm_f16(h, eps=0.0) ^ np.uint16(0x8000))


def test_gqa_gather_hand_case():
    lines = [l.split() for l in open(os.path.join(GOLDEN, "gqa_gather_hand_case.txt"))
             if l.strip() and not l.startswith("#")]
    H, Hkv, hd = map(int, lines[0])
    qkv = np.array(lines[1], np.float64)
    expect = np.array(lines[2], np.float64)
    out = oracle.gqa_gather_f16(qkv, H, Hkv, hd)
    assert np.array_equal(out, _f16_bits(expect))


def test_silu_mul_against_expit():
    g = np.array([0.0, 1.0, -1.0, 20.0, -20.0, 3.5, -0.25])
    u = np.array([5.0, 1.0, 2.0, 1.0, 1.0, -2.0, 4.0])
    out = oracle.silu_mul_f16(np.concatenate([g, u]))
    assert out[0] == 0 and out[3] == _f16_bits([20.0])[0]
    ref = _f16_bits(g * expit(g) * u)
    assert np.array_equal(out, ref)


def _identity_mat(N, K, sign=1, col_offset=0, rows=None):
    """Codes/scales with w[n][n + col_offset] = sign for n in rows, else 0."""
    codes = np.full((N, K), 8, np.uint8)
    rows = range(N) if rows is None else rows
    for n in rows:
        codes[n, n + col_offset] = 8 + sign
    s = np.ones((N, K // 32), np.float16)
    return oracle.pack(codes), s.view(np.uint16)


def _tiny_dims():
    return dict(d=32, H=2, Hkv=1, hd=16, dff=32)


def test_decode_layer_zero_weights_is_identity():
    dims = _tiny_dims()
    zero = lambda N, K: (oracle.pack(np.full((N, K), 8, np.uint8)),
                         np.ones((N, K // 32), np.uint16) * 0x3C00)
    layer = {"qkv": zero(64, 32), "o": zero(32, 32), "gate_up": zero(64, 32),
             "down": zero(32, 32)}
    h = np.random.default_rng(11).standard_normal(32)
    h0 = h.copy()
    mag = np.zeros(32)
    oracle.decode_layer(layer, dims, h, mag)
    assert np.array_equal(h, h0) and np.all(mag == 0)


def test_decode_layer_routing_hand_built():
    """Identity-shaped weights route values through each stage: the V block
    of QKV, the GQA gather, a negated O, gate|up order and down."""
    dims = _tiny_dims()
    d = 32
    qkv_codes = np.full((64, 32), 8, np.uint8)
    for n in range(16):  # V rows 48..63 pick a[0..15]; Q, K rows stay zero
        qkv_codes[48 + n, n] = 9
        qkv_codes[n, n] = 15  # Q rows are nonzero but must not reach the output
    qkv = (oracle.pack(qkv_codes), np.ones((64, 1), np.float16).view(np.uint16))
    o = _identity_mat(32, 32, sign=-1)
    gu_codes = np.full((64, 32), 8, np.uint8)
    for j in range(32):
        gu_codes[j, j] = 9         # gate = a2
        gu_codes[32 + j, j] = 7    # up = -a2
    gate_up = (oracle.pack(gu_codes), np.ones((64, 1), np.float16).view(np.uint16))
    down = _identity_mat(32, 32, sign=1)
    layer = {"qkv": qkv, "o": o, "gate_up": gate_up, "down": down}

    rng = np.random.default_rng(12)
    h0 = rng.standard_normal(d) * 3.0
    h = h0.copy()
    oracle.decode_layer(layer, dims, h)

    def rms_f16(v):
        return (v / np.sqrt(np.mean(v * v) + 1e-5)).astype(np.float16).astype(np.float64)

    a = rms_f16(h0)
    h1 = h0 - np.concatenate([a[:16], a[:16]])
    a2 = rms_f16(h1)
    mlp = (a2 * expit(a2) * -a2).astype(np.float16).astype(np.float64)
    expect = h1 + mlp
    np.testing.assert_allclose(h, expect, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- attention
# Decode attention over binary16 caches with rotary positions is not on the
# pages (the next step around the products); the pins below fix it by
# closed forms, by its reduction to the one-token stand-in at position 0,
# and by invariants of the rotation.

def test_rope_hand_case_and_invariants():
    # hd = 2: the single pair turns by pos * base^0 = pos radians
    got = oracle.rope([1.0, 0.0], 1, 10.0)
    assert np.allclose(got, [np.cos(1.0), np.sin(1.0)], rtol=0, atol=1e-15)
    # hd = 4, base 100: pair (1, 3) turns by pos * 100^(-1/2) = pos / 10
    got = oracle.rope([0.0, 1.0, 0.0, 0.0], 5, 100.0)
    assert np.allclose(got, [0.0, np.cos(0.5), 0.0, np.sin(0.5)], rtol=0, atol=1e-15)
    rng = np.random.default_rng(1)
    x = rng.standard_normal(128)
    assert np.array_equal(oracle.rope(x, 0), x)                     # position 0: identity
    y = oracle.rope(x, 37)
    pairs = lambda v: v[:64] ** 2 + v[64:] ** 2
    assert np.allclose(pairs(y), pairs(x), rtol=1e-13)              # each pair keeps its norm
    assert np.allclose(oracle.rope(oracle.rope(x, 11), 26), y, rtol=0, atol=1e-9)  # a then b = a+b


ATT_DIMS = dict(H=4, Hkv=2, hd=8)


def _qkv(rng, dims=ATT_DIMS):
    return rng.standard_normal((dims["H"] + 2 * dims["Hkv"]) * dims["hd"])


def test_attention_at_position_zero_is_the_one_token_gather():
    rng = np.random.default_rng(2)
    qkv = _qkv(rng)
    k, v = oracle.kv_cache(ATT_DIMS, 16)
    o, _ = oracle.attention(qkv, ATT_DIMS, 0, k, v)
    assert np.array_equal(oracle.f64_to_f16(o),
                          oracle.gqa_gather_f16(qkv, ATT_DIMS["H"], ATT_DIMS["Hkv"],
                                                ATT_DIMS["hd"]))


def test_attention_writes_rotated_key_and_value_rows():
    rng = np.random.default_rng(3)
    qkv = _qkv(rng)
    H, Hkv, hd = ATT_DIMS["H"], ATT_DIMS["Hkv"], ATT_DIMS["hd"]
    k, v = oracle.kv_cache(ATT_DIMS, 16)
    oracle.attention(qkv, ATT_DIMS, 9, k, v)
    for g in range(Hkv):
        kn = qkv[(H + g) * hd:(H + g + 1) * hd]
        vn = qkv[(H + Hkv + g) * hd:(H + Hkv + g + 1) * hd]
        assert np.array_equal(k[g, 9], oracle.f64_to_f16(oracle.rope(kn, 9)))
        assert np.array_equal(v[g, 9], oracle.f64_to_f16(vn))
    assert not k[:, :9].any() and not k[:, 10:].any()               # other rows untouched


def test_attention_equal_keys_average_the_values():
    rng = np.random.default_rng(4)
    qkv = _qkv(rng)
    H, Hkv, hd = ATT_DIMS["H"], ATT_DIMS["Hkv"], ATT_DIMS["hd"]
    pos = 6
    k, v = oracle.kv_cache(ATT_DIMS, 16)
    for g in range(Hkv):
        kn = qkv[(H + g) * hd:(H + g + 1) * hd]
        k[g, :pos] = oracle.f64_to_f16(oracle.rope(kn, pos))        # the key this token writes
        v[g, :pos] = oracle.f64_to_f16(rng.standard_normal((pos, hd)))
    o, mag = oracle.attention(qkv, ATT_DIMS, pos, k, v)
    for hq in range(H):
        g = hq // (H // Hkv)
        vals = oracle.f16_to_f64(v[g, :pos + 1])
        want = vals.mean(axis=0)
        assert np.allclose(o[hq * hd:(hq + 1) * hd], want, rtol=0, atol=1e-12)
        # equal weights 1 / (pos + 1): the magnitude is the mean of |v|
        assert np.allclose(mag[hq * hd:(hq + 1) * hd], np.abs(vals).mean(axis=0),
                           rtol=0, atol=1e-12)
        assert np.any(np.abs(want) < np.abs(vals).mean(axis=0) - 1e-3)  # signs differ


def test_attention_dominant_key_selects_its_value():
    rng = np.random.default_rng(5)
    H, Hkv, hd = ATT_DIMS["H"], ATT_DIMS["Hkv"], ATT_DIMS["hd"]
    pos = 3
    qkv = np.zeros((H + 2 * Hkv) * hd)
    qkv[0] = 100.0                  # query head 0 (group 0): along dim 0 before rotation
    k, v = oracle.kv_cache(ATT_DIMS, 8)
    v[0, :pos] = oracle.f64_to_f16(rng.standard_normal((pos, hd)))
    # row 1 of group 0 holds the rotated query direction, scaled: score 2^11 * 100 / sqrt(8)
    kdir = oracle.rope(np.eye(hd)[0], pos)
    k[0, 1] = oracle.f64_to_f16(kdir * 2048.0)
    o, mag = oracle.attention(qkv, ATT_DIMS, pos, k, v)
    assert np.allclose(o[:hd], oracle.f16_to_f64(v[0, 1]), rtol=0, atol=1e-12)
    # all weight on one row: the magnitude is |v| of that row
    assert np.allclose(mag[:hd], np.abs(oracle.f16_to_f64(v[0, 1])), rtol=0, atol=1e-12)
    assert np.any(oracle.f16_to_f64(v[0, 1]) < 0)


def test_attention_layer_at_position_zero_equals_stand_in_layer():
    dims = dict(d=64, H=4, Hkv=2, hd=16, dff=96)
    rng = np.random.default_rng(6)
    layer = {}
    for name, (N, K) in {"qkv": (128, 64), "o": (64, 64), "gate_up": (192, 64),
                         "down": (64, 96)}.items():
        codes = rng.integers(0, 16, (N, K), dtype=np.uint8)
        scales = oracle.f64_to_f16(np.abs(rng.standard_normal((N, K // 32))) * 0.02)
        layer[name] = (oracle.pack(codes), scales)
    h0 = rng.standard_normal(64)
    h1, m1 = h0.copy(), np.zeros(64)
    oracle.decode_layer(layer, dims, h1, m1)
    h2, m2 = h0.copy(), np.zeros(64)
    k, v = oracle.kv_cache(dims, 4)
    oracle.decode_layer_attn(layer, dims, h2, 0, k, v, m2)
    assert np.array_equal(h1, h2) and np.array_equal(m1, m2)


def _np_rms_f16(h, eps=1e-5):
    return (h / np.sqrt(np.mean(h * h) + eps)).astype(np.float16).astype(np.float64)


def _np_rotate(x, pos, base):
    """Rotate-half rotary embedding written as a complex product: the pair
    (x_i, x_{i+hd/2}) is the complex number x_i + j x_{i+hd/2}, turned by
    the angle pos * base^(-2i/hd)."""
    half = x.size // 2
    ang = pos * base ** (-2.0 * np.arange(half) / x.size)
    z = (x[:half] + 1j * x[half:]) * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag])


def _np_layer(W, dims, h, attend, eps=1e-5):
    """One decoder layer composed in numpy from dense fp64 matrices W[name];
    `attend(qkv)` returns the attention output (before rounding).  Returns
    the new residual and the magnitudes sum |w x| of the two products added
    into it."""
    from scipy.special import expit
    dff = dims["dff"]
    a = _np_rms_f16(h, eps)
    qkv = W["qkv"] @ a
    o16 = attend(qkv).astype(np.float16).astype(np.float64)
    h = h + W["o"] @ o16
    mag = np.abs(W["o"]) @ np.abs(o16)
    a2 = _np_rms_f16(h, eps)
    gu = W["gate_up"] @ a2
    m = (gu[:dff] * expit(gu[:dff]) * gu[dff:]).astype(np.float16).astype(np.float64)
    h = h + W["down"] @ m
    mag = mag + np.abs(W["down"]) @ np.abs(m)
    return h, mag


def _random_layer(rng, dims):
    d, H, Hkv, hd, dff = (dims[k] for k in ("d", "H", "Hkv", "hd", "dff"))
    shapes = {"qkv": ((H + 2 * Hkv) * hd, d), "o": (d, H * hd), "gate_up": (2 * dff, d),
              "down": (d, dff)}
    layer, dense = {}, {}
    for name, (N, K) in shapes.items():
        codes = rng.integers(0, 16, (N, K), dtype=np.uint8)
        s = (np.abs(rng.standard_normal((N, K // 32))) * 0.05).astype(np.float16)
        layer[name] = (oracle.pack(codes), s.view(np.uint16))
        dense[name] = _dense_reference(codes, s, np.zeros(K))[1]
    return layer, dense


def test_decode_layer_against_numpy_composition():
    """The stand-in layer and its magnitude output against the layer written
    out in numpy (dense matrices, numpy's float16 rounding, the GQA gather by
    slicing)."""
    dims = dict(d=64, H=4, Hkv=2, hd=16, dff=96)
    rng = np.random.default_rng(31)
    layer, W = _random_layer(rng, dims)
    H, Hkv, hd = dims["H"], dims["Hkv"], dims["hd"]

    def gather(qkv):
        V = qkv[(H + Hkv) * hd:].reshape(Hkv, hd)
        return np.repeat(V, H // Hkv, axis=0).reshape(-1)

    h0 = rng.standard_normal(64) * 2.0
    want_h, want_m = _np_layer(W, dims, h0, gather)
    h, mag = h0.copy(), np.zeros(64)
    oracle.decode_layer(layer, dims, h, mag)
    np.testing.assert_allclose(h, want_h, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mag, want_m, rtol=1e-12, atol=0)


@pytest.mark.parametrize("pos", [1, 5])
def test_attention_layer_above_position_zero_against_numpy(pos):
    """The layer with attention over caches at position pos against the same
    layer composed in numpy: rotation as a complex product, scipy's softmax
    over rows 0..pos of the group's caches (earlier rows prefilled), the new
    key and value rows written first."""
    from scipy.special import softmax
    dims = dict(d=64, H=4, Hkv=2, hd=16, dff=96)
    H, Hkv, hd = dims["H"], dims["Hkv"], dims["hd"]
    base = 10000.0
    rng = np.random.default_rng(40 + pos)
    layer, W = _random_layer(rng, dims)
    k, v = oracle.kv_cache(dims, 8)
    k[:, :pos] = rng.standard_normal((Hkv, pos, hd)).astype(np.float16).view(np.uint16)
    v[:, :pos] = rng.standard_normal((Hkv, pos, hd)).astype(np.float16).view(np.uint16)
    kn = k.view(np.float16).astype(np.float64).copy()
    vn = v.view(np.float16).astype(np.float64).copy()

    def attend(qkv):
        q = qkv[:H * hd].reshape(H, hd)
        kk = qkv[H * hd:(H + Hkv) * hd].reshape(Hkv, hd)
        vv = qkv[(H + Hkv) * hd:].reshape(Hkv, hd)
        for g in range(Hkv):
            kn[g, pos] = _np_rotate(kk[g], pos, base).astype(np.float16)
            vn[g, pos] = vv[g].astype(np.float16)
        out = np.empty((H, hd))
        for hq in range(H):
            g = hq // (H // Hkv)
            p = softmax(kn[g, :pos + 1] @ _np_rotate(q[hq], pos, base) / np.sqrt(hd))
            out[hq] = p @ vn[g, :pos + 1]
        return out.reshape(-1)

    h0 = rng.standard_normal(64) * 2.0
    want_h, want_m = _np_layer(W, dims, h0, attend)
    h, mag = h0.copy(), np.zeros(64)
    oracle.decode_layer_attn(layer, dims, h, pos, k, v, mag, base=base)
    np.testing.assert_allclose(h, want_h, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(mag, want_m, rtol=1e-10, atol=0)
    assert np.array_equal(k.view(np.float16).astype(np.float64), kn)
    assert np.array_equal(v.view(np.float16).astype(np.float64), vn)


def test_attention_two_positions_logistic_weights():
    """Two positions: the weights are the logistic function of the score
    difference, with scores (rotated q . k) / sqrt(hd); a 1/hd or unscaled
    score, or a dropped rotation of q, fails this."""
    rng = np.random.default_rng(7)
    H, Hkv, hd = ATT_DIMS["H"], ATT_DIMS["Hkv"], ATT_DIMS["hd"]
    qkv = _qkv(rng) * 2.0
    k, v = oracle.kv_cache(ATT_DIMS, 4)
    k[:, 0] = oracle.f64_to_f16(rng.standard_normal((Hkv, hd)) * 2.0)
    v[:, 0] = oracle.f64_to_f16(rng.standard_normal((Hkv, hd)))
    o, mag = oracle.attention(qkv, ATT_DIMS, 1, k, v)
    for hq in range(H):
        g = hq // (H // Hkv)
        qr = oracle.rope(qkv[hq * hd:(hq + 1) * hd], 1)
        s0 = qr @ oracle.f16_to_f64(k[g, 0]) / np.sqrt(hd)
        s1 = qr @ oracle.f16_to_f64(k[g, 1]) / np.sqrt(hd)
        p1 = 1.0 / (1.0 + np.exp(s0 - s1))
        v0, v1 = oracle.f16_to_f64(v[g, 0]), oracle.f16_to_f64(v[g, 1])
        want = (1 - p1) * v0 + p1 * v1
        assert np.allclose(o[hq * hd:(hq + 1) * hd], want, rtol=0, atol=1e-12)
        assert np.allclose(mag[hq * hd:(hq + 1) * hd], (1 - p1) * np.abs(v0) + p1 * np.abs(v1),
                           rtol=0, atol=1e-12)


# --------------------------------------------------------- quantization
def test_quantize_hand_case():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "quantize_hand_case.txt"))
            if l.strip() and not l.startswith("#")]
    w = np.zeros((1, 32), np.float32)
    want = np.full(32, 8, np.uint8)
    for i, (v, c) in enumerate(rows):
        w[0, i] = np.float32(v)
        want[i] = int(c)
    codes, s = oracle.quantize(w)
    assert oracle.f16_to_f64(s)[0, 0] == 1.0
    assert np.array_equal(codes[0], want), (codes[0], want)
    # the same values as binary16 inputs (3.49, -7.6 round; their codes do not move)
    codes16, s16 = oracle.quantize(w.astype(np.float16).view(np.uint16))
    assert np.array_equal(codes16, codes) and np.array_equal(s16, s)


def test_quantize_recovers_codes_on_the_grid():
    """Weights that are exactly s * (c - 8), with code 0 present in every
    group (so max|w| = 8 s): quantization returns the same codes and s."""
    rng = np.random.default_rng(21)
    N, K = 16, 256
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    codes.reshape(N, K // 32, 32)[:, :, 0] = 0
    s = (np.abs(rng.standard_normal((N, K // 32))) * 0.02 + 1e-3).astype(np.float16)
    w = (codes.reshape(N, K // 32, 32).astype(np.float64) - 8) * s.astype(np.float64)[..., None]
    w = w.reshape(N, K).astype(np.float32)          # exact: small integer times binary16
    got_c, got_s = oracle.quantize(w)
    assert np.array_equal(got_s, s.view(np.uint16))
    assert np.array_equal(got_c, codes)
    # and through binary16 inputs where the products are binary16 values
    s2 = np.full((N, K // 32), 0.25, np.float16)
    w2 = ((codes.astype(np.float64) - 8) * 0.25).astype(np.float16)
    c2, q2 = oracle.quantize(w2.view(np.uint16))
    assert np.array_equal(c2, codes) and np.array_equal(q2, s2.view(np.uint16))


def test_quantize_is_nearest_code_and_error_bound():
    """Brute force over all 16 codes: the chosen code is a nearest grid
    point for the stored scale, and the error is at most s/2, or the clip at
    +8 s."""
    rng = np.random.default_rng(22)
    N, K = 32, 512
    w = (rng.standard_normal((N, K)) * rng.uniform(0.01, 3.0, (N, 1))).astype(np.float32)
    codes, s = oracle.quantize(w)
    sg = np.repeat(oracle.f16_to_f64(s), 32, axis=1)
    wd = w.astype(np.float64)
    grid = (np.arange(16, dtype=np.float64) - 8)[None, None, :] * sg[..., None]
    err_all = np.abs(grid - wd[..., None])
    best = err_all.min(axis=2)
    got = np.take_along_axis(err_all, codes[..., None].astype(np.int64), axis=2)[..., 0]
    assert np.all(got == best)       # differences of exact fp64 values: no slack
    clipped = wd / sg > 7.5
    assert np.all(got[~clipped] <= sg[~clipped] * 0.5)
    # s = binary16(max|w| / 8) may sit half a binary16 ulp below max|w| / 8,
    # so w / s reaches 8 (1 + 2^-11) and the clip error s (1 + 2^-8)
    assert np.all(got[clipped] <= sg[clipped] * (1.0 + 2.0 ** -8))
    # the scale is max|w| / 8 rounded to binary16
    amax = np.abs(wd).reshape(N, K // 32, 32).max(axis=2)
    ref = (amax / 8).astype(np.float16).view(np.uint16)
    assert np.array_equal(s, ref)


def test_quantize_zero_and_tiny_groups_and_power_of_two_invariance():
    w = np.zeros((2, 64), np.float32)
    w[1, 32:] = np.float32(2.0 ** -28)          # max/8 below half the least subnormal
    codes, s = oracle.quantize(w)
    assert np.all(codes == 8) and np.all(s == 0)
    rng = np.random.default_rng(23)
    w = rng.standard_normal((8, 128)).astype(np.float32)
    c1, s1 = oracle.quantize(w)
    for k in (-3, 2, 5):
        ck, sk = oracle.quantize((w * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(ck, c1)
        assert np.array_equal(oracle.f16_to_f64(sk), oracle.f16_to_f64(s1) * 2.0 ** k)


def test_quantize_tie_goes_to_even_not_reciprocal():
    """Here w / s is exactly 3.5 (ties to even: code 12), while multiplying
    by the binary32 reciprocal of s gives just below 3.5 (code 11)."""
    s = np.float32(np.float16(1.612))
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = np.float32(8.0) * s                        # max|w| = 8 s: stored scale is s
    w[0, 1] = np.float32(float.fromhex("0x1.6928p+2"))   # 5.6430664 = 3.5 s
    q_rcp = np.rint(w[0, 1] * (np.float32(1.0) / s))
    assert q_rcp == 3.0
    codes, sc = oracle.quantize(w)
    assert oracle.f16_to_f64(sc)[0, 0] == float(s)
    assert codes[0, 0] == 15 and codes[0, 1] == 12 and np.all(codes[0, 2:] == 8)


def test_quantize_code_is_the_exactly_rounded_quotient():
    """Codes at and next to every rounding boundary, against exact rational
    arithmetic (fractions.Fraction, round-half-even): for random binary16
    scales s (normal and subnormal) and each half-integer n + 1/2, the weights
    (n + 1/2) s and its binary32 neighbours one and two steps away on either
    side.  A quotient rounded half up, truncated, or taken through a
    reciprocal fails here."""
    from fractions import Fraction
    rng = np.random.default_rng(24)
    bits = np.concatenate([rng.integers(0x0001, 0x0400, 40),      # subnormal scales
                           rng.integers(0x0400, 0x6FFF, 160)]).astype(np.uint16)
    halves = np.arange(-8, 8) + 0.5                               # n + 1/2, |.| <= 7.5
    rows = []
    for sb in bits:
        s = np.float32(np.uint16(sb).view(np.float16))
        for t in halves:
            tie = np.float32(t) * s                               # exact: few bits
            vals = [tie]
            for direction in (np.inf, -np.inf):
                v = tie
                for _ in range(2):
                    v = np.nextafter(v, np.float32(direction), dtype=np.float32)
                    vals.append(v)
            for v in vals:
                rows.append((sb, v))
    # one group per (scale, weight): w[0] = 8 s fixes the stored scale at s
    w = np.zeros((len(rows), 32), np.float32)
    for i, (sb, v) in enumerate(rows):
        s = np.float32(np.uint16(sb).view(np.float16))
        w[i, 0] = np.float32(8.0) * s
        w[i, 1] = v
    codes, sc = oracle.quantize(w)
    assert np.array_equal(sc[:, 0], np.array([r[0] for r in rows], np.uint16))
    for i, (sb, v) in enumerate(rows):
        s = Fraction(float(np.uint16(sb).view(np.float16)))
        want = min(15, max(0, round(Fraction(float(v)) / s) + 8))
        assert codes[i, 1] == want, (hex(sb), float(v), codes[i, 1], want)
    assert np.all(codes[:, 0] == 15) and np.all(codes[:, 2:] == 8)
