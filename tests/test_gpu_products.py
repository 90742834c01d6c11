"""GPU parity of q4_pack / q4_unpack / q4_gemv / q4_gemm_smallbatch against the
CPU oracle, through the C ABI.

Bar: packing bit-exact; products within |y - y_ref| <= 2e-3 * sum|w x| + 1e-6
per output.  Shapes span several tiles, ragged tails (N not a multiple of the
row tile, K not a multiple of the lane stride) and the full workload shapes.
"""
import numpy as np
import pytest
import torch

import oracle
import int4_weight_streaming_q4_amd as q4
from int4_weight_streaming_q4_amd import inputs
from helpers import DEV, assert_within, rel_err_stats, sync, u16, u8

pytestmark = pytest.mark.gpu

CFG = 1  # seeds of the single-GEMV workload


def _mat(N, K, seed, device=DEV):
    """Random packed weights + scales drawn on `device` (bytes identical for
    the oracle, which gets a host copy)."""
    packed = inputs.random_bytes(N, K, seed, device=device)
    scales = inputs.scales(N, K, seed + 1, device=device)
    return packed.to(DEV), scales.to(DEV)


def _gemv(packed, scales, x):
    y = torch.empty(packed.shape[0], dtype=torch.float32, device=DEV)
    q4.q4_gemv(packed, scales, x, y)
    sync()
    return y.cpu().numpy()


# --------------------------------------------------------------- packing
def test_pack_bit_exact_config_shape():
    codes = inputs.codes(4096, 4096, inputs.seed_of(CFG, 0, 7))
    dcodes = codes.to(DEV)
    packed = torch.empty(4096, 2048, dtype=torch.uint8, device=DEV)
    q4.q4_pack(dcodes, packed)
    sync()
    ref = oracle.pack(codes.numpy())
    assert np.array_equal(u8(packed), ref)
    back = torch.empty_like(dcodes)
    q4.q4_unpack(packed, back)
    sync()
    assert np.array_equal(u8(back), codes.numpy())


@pytest.mark.parametrize("N,K", [(1, 2), (3, 34), (65, 96), (7, 4130)])
def test_pack_ragged_and_high_bits(N, K):
    g = torch.Generator().manual_seed(N * 1000 + K)
    codes = torch.randint(0, 256, (N, K), dtype=torch.uint8, generator=g)  # high bits set
    packed = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
    q4.q4_pack(codes.to(DEV), packed)
    sync()
    assert np.array_equal(u8(packed), oracle.pack(codes.numpy()))
    back = torch.empty(N, K, dtype=torch.uint8, device=DEV)
    q4.q4_unpack(packed, back)
    sync()
    assert np.array_equal(u8(back), oracle.unpack(u8(packed)))


# --------------------------------------------------------------- gemv
def test_gemv_config1_full_parity_and_determinism():
    N = K = 4096
    codes = inputs.codes(N, K, inputs.seed_of(CFG, 0, 0))
    scales = inputs.scales(N, K, inputs.seed_of(CFG, 0, 1))
    x = inputs.act_f16(K, inputs.seed_of(CFG, 0, 2))
    packed = torch.empty(N, K // 2, dtype=torch.uint8, device=DEV)
    q4.q4_pack(codes.to(DEV), packed)
    ds, dx = scales.to(DEV), x.to(DEV)
    y1 = _gemv(packed, ds, dx)
    y2 = _gemv(packed, ds, dx)
    assert np.array_equal(y1, y2), "repeated calls must be bitwise identical"
    y_ref, mag = oracle.gemv(oracle.pack(codes.numpy()), u16(scales), u16(x))
    assert_within(y1, y_ref, mag, "config 1 gemv")
    print("config1 max/median rel err (vs sum|wx|):", rel_err_stats(y1, y_ref, mag))


@pytest.mark.parametrize("N,K", [(1, 32), (3, 96), (65, 2080), (17, 4128), (4101, 512),
                                 (130, 32768), (64, 28672)])
def test_gemv_odd_shapes(N, K):
    packed, scales = _mat(N, K, 1000 + N * 7 + K)
    x = inputs.act_f16(K, 2000 + N + K, device=DEV)
    y = _gemv(packed, scales, x)
    y_ref, mag = oracle.gemv(u8(packed), u16(scales), u16(x))
    assert_within(y, y_ref, mag, f"gemv {N}x{K}")


@pytest.mark.parametrize("rows_per_slot", [1, 2, 4])
@pytest.mark.parametrize("k_split", [1, 2, 4])
@pytest.mark.parametrize("chunks,nt", [(4, 1), (8, 0)])
def test_gemv_every_launch_shape(rows_per_slot, k_split, chunks, nt):
    N, K = 333, 1056  # ragged in rows and in chunks per lane
    packed, scales = _mat(N, K, 77)
    x = inputs.act_f16(K, 78, device=DEV)
    y = torch.empty(N, dtype=torch.float32, device=DEV)
    q4.q4_gemv_tuned(packed, scales, x, y, rows_per_slot, k_split, chunks, nt)
    sync()
    y_ref, mag = oracle.gemv(u8(packed), u16(scales), u16(x))
    assert_within(y.cpu().numpy(), y_ref, mag,
                  f"gemv R={rows_per_slot} KS={k_split} U={chunks} NT={nt}")


# Pipelined loop (chunks_in_flight == 2): the same chunks in the same order
# as the single-buffer loop, so at equal rows_per_slot and k_split the
# outputs are bitwise equal.  Shapes: a single batch per workgroup (64 x
# 1024), two and three batches per row block with ragged row counts, and
# enough row blocks that workgroups take several (even and odd counts).
@pytest.mark.parametrize("N,K,rows_per_slot,k_split", [
    (64, 1024, 1, 1), (333, 2048, 1, 1), (5001, 3072, 1, 1), (4133, 4096, 2, 2),
    (40000, 2048, 1, 1), (24577, 4096, 2, 1), (9000, 8192, 2, 4), (12289, 8192, 4, 2),
    (200, 32768, 2, 2)])
def test_gemv_pipelined_loop_bitwise(N, K, rows_per_slot, k_split):
    packed, scales = _mat(N, K, 81)
    x = inputs.act_f16(K, 82, device=DEV)
    y2 = torch.empty(N, dtype=torch.float32, device=DEV)
    y4 = torch.empty_like(y2)
    q4.q4_gemv_tuned(packed, scales, x, y2, rows_per_slot, k_split, 2, 1)
    q4.q4_gemv_tuned(packed, scales, x, y4, rows_per_slot, k_split, 4, 1)
    sync()
    assert torch.equal(y2, y4), f"pipelined != single-buffer at {N}x{K}"
    if N * K <= 24577 * 4096:
        y_ref, mag = oracle.gemv(u8(packed), u16(scales), u16(x))
        assert_within(y2.cpu().numpy(), y_ref, mag, f"pipelined gemv {N}x{K}")


def _f16(v):
    return torch.from_numpy(np.asarray(v, np.float64).astype(np.float16).view(np.int16))


@pytest.mark.parametrize("N,K", [(1, 32), (65, 2080), (333, 1056), (4133, 4096), (6144, 4096),
                                 (1000, 8192), (77, 6176), (130, 14368), (9, 28672),
                                 (260, 32768)])
def test_gemv_rows_launch_shapes_bitwise(N, K):
    """The two row-per-wave kernels that q4_gemv runs (all chunks in flight
    for K <= 4096, phases of chunks for wider K): rows per wave, chunks per
    phase and the number of workgroups (1 up to one group per wave) only
    regroup the work, so every launch shape gives q4_gemv's bits; within
    the product bound of the oracle (ragged chunk counts: K / 32 not a
    multiple of 64; a last phase shorter than the others; K at its
    maximum)."""
    packed, scales = _mat(N, K, 700 + N % 97 + K % 89)
    x = inputs.act_f16(K, 701 + K % 83, device=DEV)

    def run(fn, *shape):
        y = torch.empty(N, dtype=torch.float32, device=DEV)
        fn(packed, scales, x, y, *shape)
        sync()
        return y.cpu().numpy()

    ref = _gemv(packed, scales, x)
    y_ref, mag = oracle.gemv(u8(packed), u16(scales), u16(x))
    assert_within(ref, y_ref, mag, f"q4_gemv {N}x{K}")
    grids = (0, 1, 3, 64)
    if K <= 4096:
        for R in (2, 4):
            for grid in grids:
                assert np.array_equal(run(q4.q4_gemv_rows_tuned, R, grid), ref), (N, K, R, grid)
    else:
        y = torch.empty(N, dtype=torch.float32, device=DEV)
        with pytest.raises(q4.Q4Error, match="UNSUPPORTED"):
            q4.q4_gemv_rows_tuned(packed, scales, x, y, 2, 0)
    for R, PH in ((1, 1), (1, 2), (1, 4), (1, 7), (2, 1), (2, 2), (2, 4), (2, 7), (4, 2), (4, 4)):
        for grid in grids:
            assert np.array_equal(run(q4.q4_gemv_rowp_tuned, R, PH, grid), ref), \
                (N, K, R, PH, grid)


def test_gemv_special_values():
    N, K = 48, 256
    g = torch.Generator().manual_seed(5)
    x = inputs.act_f16(K, 9)
    dx = x.to(DEV)
    # zero point: all codes 8 -> exactly 0
    packed = torch.full((N, K // 2), 0x88, dtype=torch.uint8, device=DEV)
    scales = inputs.scales(N, K, 10).to(DEV)
    y = _gemv(packed, scales, dx)
    assert np.all(np.abs(y) <= 1e-6) and np.all(y == 0.0)
    # all codes 0 and all 15, subnormal / zero / max scales
    for byte, sbits in [(0x00, 0x0001), (0xFF, 0x03FF), (0x00, 0x0000), (0xFF, 0x7BFF),
                        (0x5A, 0x3C00)]:
        packed = torch.full((N, K // 2), byte, dtype=torch.uint8, device=DEV)
        sc = torch.full((N, K // 32), sbits, dtype=torch.int16, device=DEV)
        xs = x if sbits != 0x7BFF else _f16(np.random.default_rng(1).standard_normal(K) * 1e-3)
        y = _gemv(packed, sc, xs.to(DEV))
        y_ref, mag = oracle.gemv(u8(packed), u16(sc), u16(xs))
        assert_within(y, y_ref, mag, f"byte {byte:#x} scale {sbits:#x}")
    # impulse x: one product, exact in fp32 -> bitwise equal to the oracle
    packed, scales = _mat(N, K, 11)
    for k in (0, 1, 4, 7, 31, 32, 200, 255):
        e = np.zeros(K)
        e[k] = 1.0
        y = _gemv(packed, scales, _f16(e).to(DEV))
        y_ref, _ = oracle.gemv(u8(packed), u16(scales), u16(_f16(e)))
        assert np.array_equal(y.astype(np.float64), y_ref), k


def test_gemv_linearity_small_integers():
    N, K = 200, 1024
    packed, scales = _mat(N, K, 21)
    rng = np.random.default_rng(3)
    x1 = rng.integers(-4, 5, K).astype(np.float64)
    x2 = rng.integers(-4, 5, K).astype(np.float64)
    y1 = _gemv(packed, scales, _f16(x1).to(DEV)).astype(np.float64)
    y2 = _gemv(packed, scales, _f16(x2).to(DEV)).astype(np.float64)
    y12 = _gemv(packed, scales, _f16(x1 + x2).to(DEV)).astype(np.float64)
    _, m1 = oracle.gemv(u8(packed), u16(scales), u16(_f16(x1)))
    _, m2 = oracle.gemv(u8(packed), u16(scales), u16(_f16(x2)))
    assert np.all(np.abs(y12 - (y1 + y2)) <= 2e-3 * (m1 + m2) + 1e-6)


WORKLOAD_SHAPES = {
    "8b_qkv": (6144, 4096), "8b_o": (4096, 4096), "8b_gate_up": (28672, 4096),
    "8b_down": (4096, 14336), "70b_qkv": (10240, 8192), "70b_o": (8192, 8192),
    "70b_gate_up": (57344, 8192), "70b_down": (8192, 28672),
}


@pytest.mark.parametrize("name", list(WORKLOAD_SHAPES))
def test_gemv_workload_shapes_sampled_rows(name):
    """Full-size shapes, launched as in the decode step; every 97th row plus
    the last rows are checked one by one by the oracle."""
    N, K = WORKLOAD_SHAPES[name]
    packed, scales = _mat(N, K, inputs.seed_of(2, 0, list(WORKLOAD_SHAPES).index(name)))
    x = inputs.act_f16(K, 555, device=DEV)
    y = _gemv(packed, scales, x)
    assert np.all(np.isfinite(y))
    rows = np.unique(np.concatenate([np.arange(0, N, 97), np.arange(N - 5, N)]))
    hp = u8(packed)
    hs = u16(scales)
    y_ref, mag = oracle.gemv_rows(hp, hs, u16(x), rows)
    assert_within(y[rows], y_ref, mag, name)


# --------------------------------------------------------------- gemm
def _gemm(packed, scales, X, tuned=None):
    B = X.shape[0]
    Y = torch.empty(B, packed.shape[0], dtype=torch.float32, device=DEV)
    if tuned:
        q4.q4_gemm_tuned(packed, scales, X, Y, *tuned)
    else:
        q4.q4_gemm_smallbatch(packed, scales, X, Y)
    sync()
    return Y.cpu().numpy()


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 6, 8, 13, 16])
@pytest.mark.parametrize("N,K", [(1, 32), (17, 96), (65, 2080), (300, 1024), (33, 32768)])
def test_gemm_small_shapes(B, N, K):
    packed, scales = _mat(N, K, 300 + B + N + K)
    X = inputs.act_f16((B, K), 400 + B + K, device=DEV)
    Y = _gemm(packed, scales, X)
    Y_ref, M = oracle.gemm(u8(packed), u16(scales), u16(X))
    for b in range(B):
        assert_within(Y[b], Y_ref[b], M[b], f"gemm B={B} {N}x{K} col {b}")


GEMM_SHAPES = [(1, 4), (2, 4), (4, 4), (8, 4), (1, 8), (2, 8), (4, 8), (1, 16), (2, 16)]


@pytest.mark.parametrize("rt,nw", GEMM_SHAPES)
@pytest.mark.parametrize("K", [1184, 7584])
def test_gemm_every_launch_shape(rt, nw, K):
    """Every built launch shape (row tiles, waves) against the oracle; 37
    and 237 groups: ragged group quads, and at K = 7584 every wave runs the
    steady loop of its double buffer as well as the last quads."""
    N, B = 200, 7
    packed, scales = _mat(N, K, 900 + K % 7)
    X = inputs.act_f16((B, K), 901, device=DEV)
    Y = _gemm(packed, scales, X, tuned=(rt, nw))
    Y_ref, M = oracle.gemm(u8(packed), u16(scales), u16(X))
    for b in range(B):
        assert_within(Y[b], Y_ref[b], M[b], f"gemm rt={rt} nw={nw} K={K} col {b}")


def _lib_waves(N):
    """The row-tile launch's k split for N rows: eight waves up to one row
    tile of 16 rows per compute unit, else four (a function of the shape)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return 8 if (N + 15) // 16 <= cus else 4


@pytest.mark.parametrize("B", [5, 7, 16])
@pytest.mark.parametrize("K", [1184, 7584])
@pytest.mark.parametrize("N", [300, 4200])
def test_gemm_row_tiles_do_not_change_bits(B, K, N):
    """At a fixed k split (waves per workgroup) the row tiles per wave only
    regroup rows: every launch shape gives the same bits, and the library's
    own choice is one of them (300 rows: eight waves; 4200 rows, more than
    one row tile per compute unit: four)."""
    packed, scales = _mat(N, K, 950 + B)
    X = inputs.act_f16((B, K), 951 + B, device=DEV)
    lib = _gemm(packed, scales, X)
    for nw, rts in ((4, (2, 4, 8)), (8, (2, 4))):
        ref = _gemm(packed, scales, X, tuned=(1, nw))
        for rt in rts:
            assert np.array_equal(_gemm(packed, scales, X, tuned=(rt, nw)), ref), (rt, nw)
        if nw == _lib_waves(N):
            assert np.array_equal(lib, ref)


@pytest.mark.parametrize("N,K,B", [(16400, 4096, 16), (16384, 2048, 5), (20000, 1024, 9),
                                   (16400, 1184, 7), (16400, 32, 6), (28672, 4096, 4),
                                   (9600, 4096, 16)])
def test_gemm_activation_resident_equals_row_tiles(N, K, B):
    """With four or more row tiles per compute unit and an activation that
    fits in one workgroup's LDS the library runs the activation-resident
    launch (one workgroup per compute unit; at K = 32 three of the four k
    quarters have no quad, at K = 1184 the scales take 2-byte loads): the
    same k split and order as the row-tile launch, so the same bits, with a
    ragged last tile.  9600 rows (three tiles per unit) take the row-tile
    launch itself."""
    packed, scales = _mat(N, K, 960 + N % 97 + B)
    X = inputs.act_f16((B, K), 961 + B, device=DEV)
    ref = _gemm(packed, scales, X, tuned=(1, 4))
    got = _gemm(packed, scales, X)
    assert np.array_equal(got, ref)
    rows = np.linspace(0, N - 1, 24).astype(int)
    Y_ref, M = oracle.gemm(u8(packed)[rows], u16(scales)[rows], u16(X))
    for b in range(B):
        assert_within(got[b][rows], Y_ref[b], M[b], f"resident {N}x{K} B={B} col {b}")


def test_gemm_b1_is_gemv_and_columns_match_gemv():
    N, K = 512, 2048
    packed, scales = _mat(N, K, 31)
    X = inputs.act_f16((8, K), 32, device=DEV)
    Y1 = _gemm(packed, scales, X[:1].contiguous())
    assert np.array_equal(Y1[0], _gemv(packed, scales, X[0].contiguous()))
    Y = _gemm(packed, scales, X)
    Y_ref, M = oracle.gemm(u8(packed), u16(scales), u16(X))
    for b in range(8):
        yv = _gemv(packed, scales, X[b].contiguous())
        assert np.all(np.abs(Y[b].astype(np.float64) - yv) <= 2 * (2e-3 * M[b] + 1e-6))
    Y2 = _gemm(packed, scales, X)
    assert np.array_equal(Y, Y2)


@pytest.mark.parametrize("name", ["8b_qkv", "8b_o", "8b_gate_up", "8b_down"])
@pytest.mark.parametrize("B", [2, 4, 8, 16])
def test_gemm_workload_shapes_sampled_rows(name, B):
    N, K = WORKLOAD_SHAPES[name]
    packed, scales = _mat(N, K, inputs.seed_of(3, 0, list(WORKLOAD_SHAPES).index(name)))
    X = inputs.act_f16((B, K), inputs.seed_of(3, 0, 9) + B, device=DEV)
    Y = _gemm(packed, scales, X)
    assert np.all(np.isfinite(Y))
    rows = np.unique(np.concatenate([np.arange(0, N, 211), np.arange(N - 3, N)]))
    hp, hs, hx = u8(packed), u16(scales), u16(X)
    for b in range(B):
        y_ref, mag = oracle.gemv_rows(hp, hs, hx[b], rows)
        assert_within(Y[b][rows], y_ref, mag, f"{name} B={B} col {b}")


@pytest.mark.parametrize("B", [5, 16])
def test_gemm_special_values(B):
    """Matrix-core path (B >= 5): the codes enter the matrix op as exact
    integers and each group's scale is applied in fp32, so the all-8 zero
    point gives exactly 0, subnormal, zero and the largest binary16 scales
    stay within the product bound, and an impulse column is exact."""
    N, K = 80, 512
    X = inputs.act_f16((B, K), 930 + B, device=DEV)
    packed = torch.full((N, K // 2), 0x88, dtype=torch.uint8, device=DEV)
    scales = inputs.scales(N, K, 931).to(DEV)
    Y = _gemm(packed, scales, X)
    assert np.all(Y == 0.0)
    small = _f16(np.random.default_rng(2).standard_normal((B, K)) * 1e-3).to(DEV)
    # codes all 0 / all 15 / mixed; scales: least subnormal, largest subnormal,
    # zero, 8188 (8 * 8188 = 65504), 8192 and 65504 (the largest binary16)
    for byte, sbits in [(0x00, 0x0001), (0xFF, 0x03FF), (0x00, 0x0000), (0x00, 0x6FFF),
                        (0xFF, 0x7000), (0x00, 0x7BFF), (0x5A, 0x7BFF), (0x5A, 0x3C00)]:
        packed = torch.full((N, K // 2), byte, dtype=torch.uint8, device=DEV)
        sc = torch.full((N, K // 32), sbits, dtype=torch.int16, device=DEV)
        Xs = small if sbits >= 0x6FFF else X
        Y = _gemm(packed, sc, Xs)
        assert np.all(np.isfinite(Y)), (byte, sbits)
        Y_ref, M = oracle.gemm(u8(packed), u16(sc), u16(Xs))
        for b in range(B):
            assert_within(Y[b], Y_ref[b], M[b], f"B={B} byte {byte:#x} scale {sbits:#x} col {b}")
    # impulse columns: column b is e_k for its own k, one exact product
    packed, scales = _mat(N, K, 932)
    ks = [0, 1, 4, 7, 31, 32, 200, 255, 256, 300, 411, 480, 481, 499, 510, 511][:B]
    E = np.zeros((B, K))
    for b, k in enumerate(ks):
        E[b, k] = 1.0
    Y = _gemm(packed, scales, _f16(E).to(DEV))
    Y_ref, _ = oracle.gemm(u8(packed), u16(scales), u16(_f16(E)))
    assert np.array_equal(Y.astype(np.float64), Y_ref)


def _valu_path(B, K):
    """The library's rule: 2 <= B <= 3 columns whose binary16 copies fit 64 KB
    of LDS run the vector-ALU batch kernel; wider batches the matrix cores."""
    return 2 <= B <= 3 and B * K * 2 <= 65536


@pytest.mark.parametrize("name", ["8b_gate_up", "8b_down"])
def test_gemm_columns_independent_of_batch(name):
    """The launch shape may change with B, but no output's summation order
    does within a path: on the matrix-core path column b of a B-column
    product equals column b of the 16-column product bitwise, whatever B and
    the other columns are; on the vector-ALU path every column equals the
    single-column product (q4_gemv) bitwise."""
    N, K = WORKLOAD_SHAPES[name]
    packed, scales = _mat(N, K, inputs.seed_of(3, 1, list(WORKLOAD_SHAPES).index(name)))
    X = inputs.act_f16((16, K), inputs.seed_of(3, 1, 9), device=DEV)
    full = _gemm(packed, scales, X)
    gemv_cols = [_gemv(packed, scales, X[b].contiguous()) for b in range(4)]
    for B in (2, 3, 4, 5, 9):
        Y = _gemm(packed, scales, X[:B].contiguous())
        if _valu_path(B, K):
            for b in range(B):
                assert np.array_equal(Y[b], gemv_cols[b]), (B, b)
        else:
            assert np.array_equal(Y, full[:B]), B
    perm = torch.tensor([5, 0, 3])
    Yp = _gemm(packed, scales, X[perm].contiguous())
    if _valu_path(3, K):
        for i, b in enumerate(perm.tolist()):
            assert np.array_equal(Yp[i], _gemv(packed, scales, X[b].contiguous()))
    else:
        assert np.array_equal(Yp, full[perm.numpy()])
    perm9 = torch.tensor([8, 3, 0, 5, 1, 7, 2, 6, 4])
    assert np.array_equal(_gemm(packed, scales, X[perm9].contiguous()), full[perm9.numpy()])


# Vector-ALU batch kernel: each column is computed exactly as q4_gemv
# computes it (same unpack, same k split and order), so bitwise equal.
# Shapes: ragged rows and chunks (333 x 1056), the 8B QKV and gate+up
# widths, K = 8192 and the 8B down K (two columns fit the 64 KB stage).
@pytest.mark.parametrize("N,K", [(333, 1056), (4133, 4096), (6144, 4096), (2050, 8192),
                                 (700, 14336)])
@pytest.mark.parametrize("B", [2, 3, 4, 8])
def test_gemm_valu_columns_are_gemv(N, K, B):
    packed, scales = _mat(N, K, 91)
    X = inputs.act_f16((B, K), 92, device=DEV)
    Y = torch.empty(B, N, dtype=torch.float32, device=DEV)
    if B * K * 2 > 65536:
        # the columns do not fit the 64 KB LDS stage: refused before any launch
        with pytest.raises(q4.Q4Error, match="UNSUPPORTED"):
            q4.q4_gemm_valu(packed, scales, X, Y)
        return
    q4.q4_gemm_valu(packed, scales, X, Y)
    sync()
    Yh = Y.cpu().numpy()
    for b in range(B):
        assert np.array_equal(Yh[b], _gemv(packed, scales, X[b].contiguous())), (N, K, B, b)
    if _valu_path(B, K):
        assert np.array_equal(_gemm(packed, scales, X), Yh)
    Y_ref, M = oracle.gemm(u8(packed), u16(scales), u16(X))
    for b in (0, B - 1):
        assert_within(Yh[b], Y_ref[b], M[b], f"valu gemm {N}x{K} B={B} col {b}")
