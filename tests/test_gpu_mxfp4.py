"""GPU parity of the MXFP4 path (rotate_quant_mxfp4, mxfp4_gemm) through the
C ABI against the CPU oracle.

Codes and exponents follow tests/parity.py's check_mx: exponents agree except
where a block maximum sits on a power of two within the tie window, codes
agree except next to an E2M1 midpoint (<= 1e-4 of elements), and inputs of
the exact-arithmetic class match bit for bit.  Products: on operands whose
every partial sum is a representable fp32 (small K, narrow exponent range)
the GPU result equals the float64 sum exactly; otherwise each output is
within K * 2^-24 of the sum of the absolute terms (the fp32 accumulation
bound for K terms in any order), and dequantized outputs agree to 1e-3
relative Frobenius error.
"""
import numpy as np
import pytest

import oracle as O
import workloads as WL
from parity import Y_RTOL_FRO, check_mx, decode_nibbles, rel_fro

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import rotation_w4a4_quantization_amd as R   # raises if libw4a4.so is missing


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_mx(x, block, signs=None):
    c, e = R.rotate_quant_mxfp4(dev(x), had_block=block, signs=None if signs is None else dev(signs))
    return host(c), host(e)


def mx_codes(packed):
    """Codes of an oracle-packed operand (inputs made on the test side)."""
    return O.unpack_nibbles(packed, signed=False)


def _same_mx(packed_gpu, sbytes_gpu, ref):
    """Rows whose GPU codes and exponents equal the oracle's."""
    c = decode_nibbles(packed_gpu, signed=False) == ref["codes"]
    e = (np.asarray(sbytes_gpu, np.int64) - 127) == ref["scale_e"]
    return np.all(c, axis=1) & np.all(e, axis=1)


def abs_terms(cx, ex, cw, ew):
    """sum_k |a b| 2^(ea + eb): the oracle product on the code magnitudes."""
    return O.mx_gemm_f64(cx & 7, ex, cw & 7, ew)


def check_product(y_gpu, cx, ex, cw, ew, exact=False):
    ref = O.mx_gemm_f64(cx, ex, cw, ew)
    y = np.asarray(y_gpu, np.float64)
    if exact:
        bad = int((y != ref).sum())
        assert bad == 0, f"{bad} outputs differ from the exact sum"
        return 0.0
    K = cx.shape[1]
    bound = K * 2.0 ** -24 * abs_terms(cx, ex, cw, ew) + 1e-30
    assert np.all(np.abs(y - ref) <= bound), f"max excess {float(np.max(np.abs(y - ref) / bound))}"
    r = rel_fro(y, ref)
    assert r <= Y_RTOL_FRO
    return r


# ---------------------------------------------------------------- rotate + MXFP4
@pytest.mark.parametrize("K", [128, 384, 640, 2048, 4096, 14336, 16384])
@pytest.mark.parametrize("M", [1, 37, 300])
def test_rotate_quant_mxfp4_shapes(M, K):
    x = WL.small_random(M * 11 + K, M, K, outlier_cols=[K // 3, K - 1], mult=35.0)
    c, e = gpu_mx(x, 128)
    st = check_mx(c, e, O.rotate_mx_quant(x, 128))
    if K & (K - 1) == 0 and K > 128:
        c, e = gpu_mx(x, "full")
        st2 = check_mx(c, e, O.rotate_mx_quant(x, K))
        print(M, K, st, st2)


@pytest.mark.parametrize("K,block", [(128, 128), (1024, 128), (4096, 128), (4096, 4096),
                                     (8192, 8192), (14336, 128)])
def test_rotate_quant_mxfp4_exact_class(K, block):
    """Integer inputs: the fp32 transform is exact and y is one rounding of
    z * fl32(1/sqrt(b)) on both sides, so codes and exponents match bit for bit."""
    x = WL.exact_class(K + 3 * block, 48, K, lim=2048, outlier_cols=[7, K // 2])
    c, e = gpu_mx(x, "full" if block == K and K > 128 else 128)
    check_mx(c, e, O.rotate_mx_quant(x, block, decide="f32"), exact=True)
    check_mx(c, e, O.rotate_mx_quant(x, block))


def test_rotate_quant_mxfp4_exact_midpoints():
    """Rows x = H c (c sparse: in every 32-block one +-5, which fixes the block
    maximum, and three draws from the E2M1 midpoints).  With the full-width
    K = 1024 transform, z = H x = K c exactly, y = z / 32 = 32 c, e = 5 and
    y / 2^e = c: every non-zero element lies exactly on a midpoint, on both
    sides, so the codes pin the ties-to-even rule (and saturation-free
    rounding up to 5) bit for bit."""
    K, rows = 1024, 64
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    pos = WL.random_bytes(31, rows, 3 * (K // 32), 0, 31).astype(np.int64)
    val = WL.random_bytes(32, rows, 3 * (K // 32), 0, 13).astype(np.int64)
    c = np.zeros((rows, K))
    for r in range(rows):
        for j in range(K // 32):
            c[r, 32 * j + (r + j) % 32] = 5.0 if (r + j) % 2 else -5.0
            for u in range(3):
                p_ = 32 * j + (((r + j) % 32) + 1 + pos[r, 3 * j + u] % 31) % 32
                v_ = mids[val[r, 3 * j + u] % 7] * (1.0 if val[r, 3 * j + u] < 7 else -1.0)
                c[r, p_] = v_
    x64 = O.rotate(c, K)                       # H c (the unnormalized transform)
    x = x64.astype(np.float16)
    assert np.array_equal(x.astype(np.float64), x64), "H c must be exact in fp16"
    ref = O.rotate_mx_quant(x, K, decide="f32")
    assert np.all(ref["scale_e"] == 5)
    t = ref["y"] / 32.0
    assert np.array_equal(t, c)
    # 1/sqrt(1024) is a power of two, so the float64 definition gives the same y
    assert np.array_equal(O.rotate_mx_quant(x, K)["y"], ref["y"])
    n_ties = int(np.isin(np.abs(t), mids).sum())
    assert n_ties >= 3 * rows * (K // 32)
    cg, eg = gpu_mx(x, "full")
    st = check_mx(cg, eg, ref, exact=True)
    print("exact midpoints", n_ties, st)


@pytest.mark.parametrize("block", [128, "full"])
def test_rotate_quant_mxfp4_signs(block):
    K = 2048
    x = WL.small_random(321, 64, K, outlier_cols=[9, 1500], mult=30.0)
    d = WL.hadamard_signs(K, seed=4)
    b = 128 if block == 128 else K
    c, e = gpu_mx(x, block, signs=d)
    check_mx(c, e, O.rotate_mx_quant(x, b, signs=d))


def test_rotate_quant_mxfp4_edge_rows():
    K = 512
    x = np.zeros((6, K), np.float16)
    x[1] = 3.0                                  # constant row: one nonzero per 128-block
    x[2, 17] = -60000.0                         # one-hot, near the fp16 maximum
    x[3] = np.float16(6e-8)                     # fp16 subnormals
    x[4, ::2] = 1.0
    x[4, 1::2] = -1.0
    x[5] = WL.small_random(9, 1, K)[0]
    for block in (128, "full"):
        b = 128 if block == 128 else K
        c, e = gpu_mx(x, block)
        check_mx(c, e, O.rotate_mx_quant(x, b))
        assert np.all(e[0] == 0) and np.all(c[0] == 0)     # a zero block: byte 0, zero codes


def test_rotate_quant_mxfp4_stride_and_empty():
    x = WL.small_random(12, 40, 1024 + 64, outlier_cols=[3], mult=40.0)
    c1, e1 = R.rotate_quant_mxfp4(dev(x)[:, :1024], 128)          # ldx = 1088 > K
    c2, e2 = R.rotate_quant_mxfp4(dev(np.ascontiguousarray(x[:, :1024])), 128)
    assert torch.equal(c1, c2) and torch.equal(e1, e2)
    c, e = R.rotate_quant_mxfp4(torch.empty((0, 256), dtype=torch.float16, device="cuda"), 128)
    assert c.shape == (0, 128) and e.shape == (0, 8)


@pytest.mark.parametrize("cfg,block", [("qproj", 128), ("qproj", 4096), ("downproj", 128)])
def test_rotate_quant_mxfp4_full_size(cfg, block):
    """Full-size launch; every q_proj row, and 1024 seeded down_proj rows in
    chunks (rows are independent), checked against the oracle."""
    x = WL.qproj(with_w=False)["X"] if cfg == "qproj" else WL.downproj(with_w=False)["X"]
    c, e = gpu_mx(x, block)
    if cfg == "qproj":
        rows = np.arange(x.shape[0])
    else:
        rows = np.sort(np.random.default_rng(5).choice(x.shape[0], 1024, replace=False))
    b = 128 if block == 128 else x.shape[1]
    flips = 0
    for k in range(0, len(rows), 256):
        r = rows[k:k + 256]
        flips += check_mx(c[r], e[r], O.rotate_mx_quant(x[r], b))["flips"]
    print(cfg, block, "rows", len(rows), "flips", flips)


# ---------------------------------------------------------------- MXFP4 GEMM
GEMM_SHAPES = [(1, 16, 256), (4, 130, 384), (16, 64, 128), (17, 200, 256), (100, 130, 384),
               (300, 256, 256), (600, 384, 256), (1000, 200, 384), (513, 129, 128)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_mxfp4_gemm_exact(M, N, K):
    """Random codes (all 16, -0 included) with exponents in [-2, 2]: every
    partial sum is a multiple of 2^-6 below 2^18, so fp32 holds it exactly and
    the GPU result must equal the float64 sum bit for bit."""
    s = M * 7 + N * 3 + K
    px, pw = WL.random_bytes(s, M, K // 2), WL.random_bytes(s + 1, N, K // 2)
    bx, bw = WL.random_bytes(s + 2, M, K // 32, 125, 129), WL.random_bytes(s + 3, N, K // 32, 125, 129)
    y = host(R.mxfp4_gemm(dev(px), dev(bx), dev(pw), dev(bw)))
    check_product(y, mx_codes(px), bx.astype(np.int64) - 127, mx_codes(pw), bw.astype(np.int64) - 127,
                  exact=True)


@pytest.mark.parametrize("M,N,K", [(8, 300, 4096), (300, 256, 4096), (700, 260, 2176), (64, 128, 14336)])
def test_mxfp4_gemm_rounding_bound(M, N, K):
    s = M + N + K
    px, pw = WL.random_bytes(s, M, K // 2), WL.random_bytes(s + 1, N, K // 2)
    bx, bw = WL.random_bytes(s + 2, M, K // 32, 117, 137), WL.random_bytes(s + 3, N, K // 32, 117, 137)
    y = host(R.mxfp4_gemm(dev(px), dev(bx), dev(pw), dev(bw)))
    r = check_product(y, mx_codes(px), bx.astype(np.int64) - 127, mx_codes(pw), bw.astype(np.int64) - 127)
    print(M, N, K, "rel_fro", r)


@pytest.mark.parametrize("M,N,K,exact", [(2048, 4096, 256, True), (2048, 4096, 384, True),
                                         (2048, 4096, 768, False), (2048, 4096, 1152, False),
                                         (2304, 4096, 640, False)])
def test_mxfp4_gemm_one_tile_per_cu(M, N, K, exact):
    """The 256-row instance (one or more tiles per CU) over full groups of four
    K-steps and partial last groups of 1, 2 and 3 steps (K/128 = 2, 3, 6, 9, 5),
    checked on sampled rows
    that include the first and last row of every 256-row tile: exactly for
    K <= 384 with exponents in [-2, 2], else to the fp32 accumulation bound."""
    s = M + 3 * N + K
    px, pw = WL.random_bytes(s, M, K // 2), WL.random_bytes(s + 1, N, K // 2)
    lo, hi = (125, 129) if exact else (117, 137)
    bx, bw = WL.random_bytes(s + 2, M, K // 32, lo, hi), WL.random_bytes(s + 3, N, K // 32, lo, hi)
    y = host(R.mxfp4_gemm(dev(px), dev(bx), dev(pw), dev(bw)))
    edges = np.concatenate([np.arange(0, M, 256), np.minimum(np.arange(255, M + 255, 256), M - 1)])
    rest = np.random.default_rng(s).choice(M, 256 - len(np.unique(edges)), replace=False)
    rows = np.unique(np.concatenate([edges, rest]))
    r = check_product(y[rows], mx_codes(px[rows]), bx[rows].astype(np.int64) - 127, mx_codes(pw),
                      bw.astype(np.int64) - 127, exact=exact)
    print(M, N, K, "rows", len(rows), "rel_fro", r)


def test_mxfp4_gemm_output_stride():
    M, N, K = 40, 96, 256
    px, pw = WL.random_bytes(1, M, K // 2), WL.random_bytes(2, N, K // 2)
    bx, bw = WL.random_bytes(3, M, K // 32, 126, 128), WL.random_bytes(4, N, K // 32, 126, 128)
    big = torch.full((M, N + 36), 7.0, dtype=torch.float32, device="cuda")
    R.mxfp4_gemm(dev(px), dev(bx), dev(pw), dev(bw), out=big[:, :N])
    y = host(big)
    assert np.all(y[:, N:] == 7.0)            # columns past N are not written
    check_product(y[:, :N], mx_codes(px), bx.astype(np.int64) - 127, mx_codes(pw), bw.astype(np.int64) - 127,
                  exact=True)



@pytest.mark.parametrize("M,N,K,pad", [(40, 100, 256, 3), (2048, 4096, 128, 1), (600, 260, 256, 2)])
def test_mxfp4_gemm_output_stride_unaligned(M, N, K, pad):
    """Unaligned row stride and ragged N take the scalar stores of the output
    epilogue (64-row and 256-row tilings); exact-class inputs, so the values
    must still equal the float64 product bit for bit."""
    s = 31 * M + N + pad
    px, pw = WL.random_bytes(s, M, K // 2), WL.random_bytes(s + 1, N, K // 2)
    bx, bw = WL.random_bytes(s + 2, M, K // 32, 126, 128), WL.random_bytes(s + 3, N, K // 32, 126, 128)
    big = torch.full((M, N + pad), 7.0, dtype=torch.float32, device="cuda")
    R.mxfp4_gemm(dev(px), dev(bx), dev(pw), dev(bw), out=big[:, :N])
    y = host(big)
    assert np.all(y[:, N:] == 7.0)
    check_product(y[:, :N], mx_codes(px), bx.astype(np.int64) - 127, mx_codes(pw), bw.astype(np.int64) - 127,
                  exact=True)

def test_mxfp4_gemm_empty():
    z = torch.empty((0, 64), dtype=torch.uint8, device="cuda")
    ze = torch.empty((0, 4), dtype=torch.uint8, device="cuda")
    w = torch.zeros((8, 64), dtype=torch.uint8, device="cuda")
    we = torch.zeros((8, 4), dtype=torch.uint8, device="cuda")
    y = R.mxfp4_gemm(z, ze, w, we)
    assert y.shape == (0, 8)


# ---------------------------------------------------------------- end to end
@pytest.mark.parametrize("cfg", ["tiny", "qproj", "downproj", "gateup"])
def test_mxfp4_linear_end_to_end(cfg):
    """X and W rotated and quantized to MXFP4 on the GPU, then multiplied:
    the product agrees with the oracle's whole pipeline to 1e-3 relative
    Frobenius error, and with the oracle's product of the GPU's own codes to
    the fp32 accumulation bound."""
    if cfg == "tiny":
        d = WL.tiny()
        X, W = d["X"], d["W"]
        rows, cols = np.arange(X.shape[0]), np.arange(W.shape[0])
    else:
        # full-size GEMM (the 8-wave 256-row instance from 512 tiles up, the
        # 16-wave one below), checked on sampled rows and columns
        if cfg == "qproj":
            X, W = WL.qproj(with_w=False)["X"], WL.qproj_weight()
        else:
            d = WL.downproj() if cfg == "downproj" else WL.gateup()
            X, W = d["X"], d["W"]
            del d
        rng = np.random.default_rng(6)
        rows = np.sort(rng.choice(X.shape[0], 64, replace=False))
        cols = np.sort(rng.choice(W.shape[0], 256, replace=False))
    cx, ex = R.rotate_quant_mxfp4(dev(X), 128)
    cw, ew = R.rotate_quant_mxfp4(dev(W), 128)
    y = host(R.mxfp4_gemm(cx, ex, cw, ew))[np.ix_(rows, cols)]
    ax, aw = O.rotate_mx_quant(X[rows], 128), O.rotate_mx_quant(W[cols], 128)
    # rows and columns whose GPU codes and exponents equal the oracle's: the
    # product there is the oracle's product of its own codes to the fp32 bound
    rx = _same_mx(host(cx)[rows], host(ex)[rows], ax)
    rw = _same_mx(host(cw)[cols], host(ew)[cols], aw)
    assert rx.mean() > 0.9 and rw.mean() > 0.9
    check_product(y[np.ix_(rx, rw)], ax["codes"][rx], ax["scale_e"][rx], aw["codes"][rw], aw["scale_e"][rw])
    ref = O.mx_gemm_f64(ax["codes"], ax["scale_e"], aw["codes"], aw["scale_e"])
    r = rel_fro(y, ref)
    exact = np.asarray(X[rows], np.float64) @ np.asarray(W[cols], np.float64).T
    print(cfg, "rel_fro vs oracle", r, "MXFP4 error vs X W^T", rel_fro(y, exact))
    assert r <= Y_RTOL_FRO
