"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test checks the oracle against something the pages or mathematics fix:
hand-computed worked examples (tests/golden), closed forms, invariants,
brute force on tiny inputs, and sampling-error-bounded statistics.  Pages:
  "Rotations for 4-Bit Activations: QuaRot, SpinQuant, and Friends" [ROT]
  "SpinQuant (learned rotations + W4A4KV4)" record [SQ]
  "QuaRot (rotation-based outlier removal, W4A4KV4)" record [QR]
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------- Hadamard
def test_hadamard_matches_hand_written_h8():
    rows = _golden_lines("hadamard8.txt")
    ref = np.array([[1 if c == "+" else -1 for c in r.split()] for r in rows])
    assert np.array_equal(O.hadamard(8), ref)
    assert np.array_equal(O.hadamard(2), np.array([[1, 1], [1, -1]]))
    assert np.array_equal(O.hadamard(1), np.array([[1]]))


@pytest.mark.parametrize("n", [2, 4, 16, 128, 512, 1024])
def test_hadamard_entries_closed_form(n):
    """Sylvester's H has h_ij = (-1)^popcount(i & j) (textbook closed form)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    assert np.array_equal(O.hadamard(n), np.where(pc % 2 == 0, 1, -1))


@pytest.mark.parametrize("n", [1, 2, 8, 128, 1024])
def test_hadamard_orthogonal(n):
    """H H^T = n I exactly, so Q = H / sqrt(n) is orthogonal ([ROT] invariance needs Q Q^T = I)."""
    h = O.hadamard(n).astype(np.float64)
    assert np.array_equal(h @ h.T, n * np.eye(n))
    assert np.array_equal(h, h.T)


@pytest.mark.parametrize("n", [2048, 4096, 16384])
def test_hadamard_large_sampled_entries(n):
    h = O.hadamard(n)
    rng = np.random.default_rng(n)
    ii = rng.integers(0, n, 2000)
    jj = rng.integers(0, n, 2000)
    want = [(-1) ** bin(int(a) & int(b)).count("1") for a, b in zip(ii, jj)]
    assert np.array_equal(h[ii, jj], np.array(want))


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        O.hadamard(12)


# ---------------------------------------------------------------- rotation
def test_fwht_worked_examples():
    for ln in _golden_lines("worked_examples.txt"):
        if not ln.startswith("fwht"):
            continue
        head, xs, zs = [p.strip() for p in ln.split("|")]
        n = int(head.split()[1])
        x = np.array([float(v) for v in xs.split()])[None, :]
        z = np.array([float(v) for v in zs.split()])
        assert x.shape[1] == n
        assert np.array_equal(O.rotate(x, n)[0], z), ln


def _butterfly(v):
    """Independent recursive fast Walsh-Hadamard transform on Python ints/Fractions."""
    n = len(v)
    if n == 1:
        return list(v)
    a = _butterfly(v[: n // 2])
    b = _butterfly(v[n // 2:])
    return [p + q for p, q in zip(a, b)] + [p - q for p, q in zip(a, b)]


@pytest.mark.parametrize("block", [2, 8, 32, 128])
def test_rotate_equals_exact_butterfly(block):
    """The dense float64 product equals an exact rational butterfly, bit for bit."""
    x = WL.small_random(1, 3, 2 * block, outlier_cols=[1], mult=40.0)
    z = O.rotate(x, block)
    for r in range(3):
        for b0 in range(0, 2 * block, block):
            exact = _butterfly([Fraction(float(v)) for v in x[r, b0:b0 + block]])
            assert [Fraction(float(v)) for v in z[r, b0:b0 + block]] == exact


@pytest.mark.parametrize("block", [128, 4096])
def test_invariance_xwT(block):
    """[ROT] "A rotation changes nothing": X W^T = (XQ)(WQ)^T, to 1e-10 in float64."""
    x = WL.qproj(M=256, with_w=False)["X"].astype(np.float64)
    w = WL.small_random(2, 256, 4096, std=0.02).astype(np.float64)
    ref = x @ w.T
    rot = O.rotate_normalized(x, block) @ O.rotate_normalized(w, block).T
    assert np.linalg.norm(ref - rot) / np.linalg.norm(ref) < 1e-10


@pytest.mark.parametrize("block", [1, 128, 1024])
def test_involution_and_parseval(block):
    x = WL.small_random(3, 8, 2048, outlier_cols=[5], mult=30.0).astype(np.float64)
    y = O.rotate_normalized(x, block)
    assert np.allclose(O.rotate_normalized(y, block), x, rtol=0, atol=1e-12)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


@pytest.mark.parametrize("n,j,m", [(128, 3, 50.0), (128, 77, -50.0), (4096, 1234, 30.0)])
def test_outlier_spreads_evenly(n, j, m):
    """[ROT] "A rotation changes nothing": an outlier M in channel j becomes
    +-M/sqrt(n) in every channel, the sign being H's row j."""
    x = np.zeros((1, n))
    x[0, j] = m
    y = O.rotate_normalized(x, n)[0]
    pc = np.array([bin(j & i).count("1") for i in range(n)])
    assert np.allclose(y, m / math.sqrt(n) * np.where(pc % 2 == 0, 1, -1), rtol=1e-15, atol=0)
    for mode in ("f64", "f32"):
        q = O.quant_sym_rows(O.rotate(x, n), n, mode)
        assert np.array_equal(q["codes"][0], 7 * np.sign(m) * np.where(pc % 2 == 0, 1, -1))
    # s = max|y| / 7 = |M| / (7 sqrt(n)); in the fp32 form one division of fp32 values
    assert math.isclose(O.quant_sym_rows(O.rotate(x, n), n)["scale"][0], abs(m) / (7 * math.sqrt(n)),
                        rel_tol=4e-16)
    assert q["scale"][0] == np.float32(abs(m)) / np.float32(7 * math.sqrt(n))


def test_constant_row_concentrates():
    """A constant row c.1 rotates to c*b at index 0 of every block, zeros elsewhere."""
    x = np.full((1, 512), -3.0)
    z = O.rotate(x, 128)[0].reshape(4, 128)
    assert np.all(z[:, 0] == -3.0 * 128) and np.all(z[:, 1:] == 0)
    q = O.quant_sym_rows(z.reshape(1, -1), 128)["codes"].reshape(4, 128)
    assert np.all(q[:, 0] == -7) and np.all(q[:, 1:] == 0)


def test_rotation_of_fp16_is_exact_integer_multiple():
    """fp16 inputs: z * 2^24 is an integer below 2^53 (the rotation is exact)."""
    x = WL.qproj(M=64, with_w=False)["X"]
    z = O.rotate(x, 4096) * 2.0 ** 24
    assert np.all(z == np.rint(z)) and np.abs(z).max() < 2.0 ** 53


# ---------------------------------------------------------------- quantizers
def test_quant_worked_examples():
    for ln in _golden_lines("worked_examples.txt"):
        kind = ln.split("|")[0].strip()
        if kind == "sym":
            _, zs, qs, ss, bs = [p.strip() for p in ln.split("|")]
            z = np.array([[float(v) for v in zs.split()]])
            for mode in ("f64", "f32"):
                d = O.quant_sym_rows(z, 1, mode)
                assert d["codes"][0].tolist() == [int(v) for v in qs.split()], ln
                assert d["scale"][0] == float(ss), ln
                assert O.pack_nibbles(d["codes"])[0].tolist() == [int(b, 16) for b in bs.split()], ln
        elif kind == "asym":
            _, zs, qs, ss, zps = [p.strip() for p in ln.split("|")]
            z = np.array([[float(v) for v in zs.split()]])
            for mode in ("f64", "f32"):
                d = O.quant_asym_groups(z, 1, group=z.shape[1], mode=mode)
                assert d["codes"][0].tolist() == [int(v) for v in qs.split()], ln
                assert d["scale"][0, 0] == float(ss), ln
                assert d["zp"][0, 0] == int(zps), ln


def _brute_code(t, lo, hi):
    """Nearest integer in [lo, hi] to t, ties to the even one (exhaustive search)."""
    best = None
    for q in range(lo, hi + 1):
        key = (abs(Fraction(t) - q), q % 2)
        if best is None or key < best[0]:
            best = (key, q)
    return best[1]


def test_sym_codes_brute_force():
    """Codes of the float64 mode = the nearest level to the exact rational
    7 z / max|z| (z exact for fp16 inputs), by exhaustive search in Fraction."""
    x = WL.small_random(4, 6, 256, outlier_cols=[9], mult=50.0)
    z = O.rotate(x, 128)
    d = O.quant_sym_rows(z, 128)
    for r in range(6):
        zr = [Fraction(float(v)) for v in z[r]]
        a = max(abs(v) for v in zr)
        for k in range(256):
            assert d["codes"][r, k] == _brute_code(7 * zr[k] / a, -7, 7)
        assert d["scale"][r] == float(a) / (7 * math.sqrt(128))


def test_asym_levels_brute_force():
    """Zero-points and codes of the float64 mode from the exact rationals
    -15 lo / r and 15 z / r, r = hi - lo with the range widened to include 0."""
    z = O.rotate(WL.small_random(5, 4, 256, outlier_cols=[2], mult=20.0), 128)
    d = O.quant_asym_groups(z, 128)
    for r in range(4):
        for g in range(2):
            grp = [Fraction(float(v)) for v in z[r, g * 128:(g + 1) * 128]]
            lo, hi = min(min(grp), Fraction(0)), max(max(grp), Fraction(0))
            rng_ = hi - lo
            zp = int(d["zp"][r, g])
            assert zp == _brute_code(-15 * lo / rng_, 0, 15)
            for k in range(128):
                lvl = _brute_code(15 * grp[k] / rng_, -100, 100)
                assert d["codes"][r, g * 128 + k] == min(max(lvl + zp, 0), 15)


def _dist_to_tie(t):
    return np.abs(np.abs(t - np.floor(t)) - 0.5)


# fp32 rounding budget of the exact-fp32 form against the definition: the
# symmetric t32 = fl32(z) * fl32(7 / fl32(a)) carries three relative
# roundings of at most 2^-24 each; the asymmetric one four (fl32 of z, of hi
# or lo, of hi - lo, of 15 / r).  The float64 evaluation adds a few 2^-53.
SYM_T_BUDGET = 3.001 * 2.0 ** -24
ASYM_T_BUDGET = 4.001 * 2.0 ** -24


def test_decision_modes_at_an_exact_tie():
    """Hand-worked: z = (42, 3), block 1.  The definition gives t = 7*3/42 = 1/2
    exactly, which rounds half to even: code 0.  The exact-fp32 form uses
    fl32(7/42) = fl32(1/6) = 11184811 * 2^-26 > 1/6, so t32 = 3 * that > 1/2
    and the code is 1 (-1 for z = -3).  This is the only kind of place where
    the two modes may differ, and the GPU-vs-oracle tie window covers it."""
    z = np.array([[42.0, 3.0], [42.0, -3.0]])
    d64, d32 = O.quant_sym_rows(z, 1), O.quant_sym_rows(z, 1, "f32")
    assert d64["t"][0, 1] == 0.5 and d64["codes"].tolist() == [[7, 0], [7, 0]]
    assert np.float32(1 / 6) == np.float32(11184811 * 2.0 ** -26)
    assert d32["t"][0, 1] == 3 * 11184811 * 2.0 ** -26 and d32["codes"].tolist() == [[7, 1], [7, -1]]


@pytest.mark.parametrize("cfg,block", [("qproj", 128), ("qproj", 4096), ("downproj", 128)])
def test_decision_modes_agree_off_ties_sym(cfg, block):
    """The exact-fp32 form decides every code as the float64 definition does,
    except within its rounding budget (|t| * 3 * 2^-24 <= 1.26e-6) of a .5
    tie; the scales agree to 3 fp32 roundings."""
    x = (WL.qproj(M=512, with_w=False) if cfg == "qproj" else WL.downproj(M=192, with_w=False))["X"]
    z = O.rotate(x, block)
    d64, d32 = O.quant_sym_rows(z, block), O.quant_sym_rows(z, block, "f32")
    diff = d64["codes"] != d32["codes"]
    assert np.all(np.abs(d64["t"] - d32["t"]) <= np.abs(d64["t"]) * SYM_T_BUDGET)
    assert np.all(_dist_to_tie(d64["t"][diff]) <= np.abs(d64["t"][diff]) * SYM_T_BUDGET)
    assert np.all(np.abs(d64["codes"].astype(int) - d32["codes"])[diff] == 1)
    assert np.all(np.abs(d32["scale"] - d64["scale"]) <= 3.001 * 2.0 ** -24 * d64["scale"])


def test_decision_modes_agree_off_ties_asym():
    x = WL.gateup(M=96, with_w=False)["X"]
    z = O.rotate(x, 128)
    d64, d32 = O.quant_asym_groups(z, 128), O.quant_asym_groups(z, 128, mode="f32")
    assert np.all(np.abs(d64["t"] - d32["t"]) <= np.abs(d64["t"]) * ASYM_T_BUDGET)
    assert np.all(np.abs(d64["t_zp"] - d32["t_zp"]) <= np.abs(d64["t_zp"]) * ASYM_T_BUDGET)
    zdiff = d64["zp"] != d32["zp"]
    assert np.all(_dist_to_tie(d64["t_zp"][zdiff]) <= np.abs(d64["t_zp"][zdiff]) * ASYM_T_BUDGET)
    lv64 = d64["codes"].astype(int).reshape(96, 64, 128) - d64["zp"][:, :, None]
    lv32 = d32["codes"].astype(int).reshape(96, 64, 128) - d32["zp"][:, :, None]
    diff = (lv64 != lv32).reshape(96, -1)
    near = _dist_to_tie(d64["t"]) <= np.abs(d64["t"]) * ASYM_T_BUDGET
    near |= np.repeat(zdiff, 128, axis=1)
    assert np.all(near[diff])


def test_decision_modes_agree_off_ties_mx():
    """MXFP4: y32 = fl32(fl32(z) * fl32(1/sqrt(b))) is within 3 fp32 roundings
    of z / sqrt(b); exponents differ only where the block maximum is that close
    to a power of two, codes only that close to an E2M1 midpoint."""
    x = WL.qproj(M=256, with_w=False)["X"]
    for block in (128, 4096):
        d64, d32 = O.rotate_mx_quant(x, block), O.rotate_mx_quant(x, block, decide="f32")
        assert np.all(np.abs(d64["y"] - d32["y"]) <= np.abs(d64["y"]) * SYM_T_BUDGET)
        ediff = d64["scale_e"] != d32["scale_e"]
        amax = np.abs(d64["y"].reshape(256, -1, 32)).max(axis=-1)
        lg = np.log2(amax)
        assert np.all(np.abs(lg - np.round(lg))[ediff] <= 2 * SYM_T_BUDGET)
        t = d64["y"].reshape(256, -1, 32) / np.exp2(d64["scale_e"])[..., None]
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
        near = (np.abs(np.abs(t)[..., None] - mids) <= mids * SYM_T_BUDGET).any(axis=-1)
        near |= np.repeat(ediff[..., None], 32, axis=-1)
        cdiff = (d64["codes"] != d32["codes"]).reshape(near.shape)
        assert np.all(near[cdiff])


@pytest.mark.parametrize("block", [128, 4096])
def test_sym_quant_invariants(block):
    x = WL.qproj(M=32, with_w=False)["X"]
    z = O.rotate(x, block)
    d = O.quant_sym_rows(z, block)
    q, s = d["codes"].astype(np.int64), d["scale"].astype(np.float64)
    y = z / math.sqrt(block)
    assert q.min() >= -7 and q.max() <= 7
    # no clipping: every element within half a step (fp32 slack on the scale)
    assert np.all(np.abs(y - q * s[:, None]) <= 0.5 * s[:, None] * (1 + 1e-5))
    # the largest element lands on +-7 with its own sign
    am = np.argmax(np.abs(z), axis=1)
    assert np.array_equal(q[np.arange(32), am], 7 * np.sign(z[np.arange(32), am]))
    # scale ~ max|y| / 7 to fp32 accuracy
    assert np.allclose(s, np.abs(y).max(axis=1) / 7, rtol=3e-7, atol=0)
    # odd symmetry and power-of-two scale invariance
    dn = O.quant_sym_rows(-z, block)
    assert np.array_equal(dn["codes"], -d["codes"])
    d2 = O.quant_sym_rows(z * 8, block)
    assert np.array_equal(d2["codes"], d["codes"]) and np.array_equal(d2["scale"], d["scale"] * 8)
    # monotone along each row
    for r in range(4):
        o = np.argsort(z[r], kind="stable")
        assert np.all(np.diff(q[r, o]) >= 0)


def test_asym_quant_invariants():
    x = WL.gateup(M=16, with_w=False)["X"]
    z = O.rotate(x, 128)
    d = O.quant_asym_groups(z, 128)
    q = d["codes"].astype(np.int64).reshape(16, 64, 128)
    zp = d["zp"].astype(np.int64)
    s = d["scale"].astype(np.float64)
    y = (z / math.sqrt(128)).reshape(16, 64, 128)
    assert q.min() >= 0 and q.max() <= 15 and zp.max() <= 15
    yh = (q - zp[:, :, None]) * s[:, :, None]
    assert np.all(np.abs(y - yh) <= 0.5 * s[:, :, None] * (1 + 1e-5))
    # the group minimum (when negative) maps to code 0 exactly
    mn = y.min(axis=2)
    idx = np.argmin(y, axis=2)
    got = np.take_along_axis(q, idx[:, :, None], axis=2)[:, :, 0]
    assert np.all(got[mn < 0] == 0)


def test_zero_rows_and_groups():
    z = np.zeros((2, 256))
    d = O.quant_sym_rows(z, 128)
    assert np.all(d["codes"] == 0) and np.all(d["scale"] == 0)
    a = O.quant_asym_groups(z, 128)
    assert np.all(a["codes"] == 0) and np.all(a["scale"] == 0) and np.all(a["zp"] == 0)


# ---------------------------------------------------------------- packing
def test_pack_all_nibble_pairs():
    lo, hi = np.meshgrid(np.arange(16), np.arange(16))            # lo varies fastest
    q = np.stack([lo.ravel(), hi.ravel()], axis=1)
    p = O.pack_nibbles(q)[:, 0]
    assert np.array_equal(p, np.arange(256, dtype=np.uint8))      # lo + 16 hi enumerates 0..255
    assert np.array_equal(O.unpack_nibbles(p[:, None], signed=False), q)
    s = np.array([[-7, 7], [-1, -1], [7, -7], [0, -3]])
    assert O.pack_nibbles(s)[:, 0].tolist() == [0x79, 0xFF, 0x97, 0xD0]
    assert np.array_equal(O.unpack_nibbles(O.pack_nibbles(s), signed=True), s)


# ---------------------------------------------------------------- integer GEMM and epilogues
def test_int_gemm_brute_force():
    rng = np.random.default_rng(9)
    a = rng.integers(-7, 8, (5, 256))
    b = rng.integers(-7, 8, (6, 256))
    got = O.int_gemm(a, b)
    for m in range(5):
        for n in range(6):
            assert got[m, n] == sum(int(a[m, k]) * int(b[n, k]) for k in range(256))
    big = np.full((1, 14336), -7)
    assert O.int_gemm(big, big)[0, 0] == 49 * 14336


def test_epilogue_closed_forms():
    acc = np.array([[3, -5], [0, 702464]])
    ones = np.ones(2, np.float32)
    assert np.array_equal(O.epilogue_sym_f32(acc, ones, ones), acc.astype(np.float32))
    sx = np.array([0.5, 2.0], np.float32)
    sw = np.array([0.25, 4.0], np.float32)
    want = np.array([[0.375, -10.0], [0.0, 702464.0 * 8]], np.float32)
    assert np.array_equal(O.epilogue_sym_f32(acc, sx, sw), want)


def test_asym_gemm_brute_force():
    rng = np.random.default_rng(10)
    M, N, K = 3, 4, 256
    u = rng.integers(0, 16, (M, K))
    zp = rng.integers(0, 16, (M, K // 128))
    qw = rng.integers(-7, 8, (N, K))
    sx = rng.random((M, K // 128)).astype(np.float32)
    sw = rng.random(N).astype(np.float32)
    got = O.gemm_asym_f64(u, zp, sx, qw, sw)
    gs = O.group_sums(qw)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for g in range(K // 128):
                dot = sum(int(u[m, k]) * int(qw[n, k]) for k in range(g * 128, g * 128 + 128))
                tot += Fraction(float(sx[m, g])) * (dot - int(zp[m, g]) * int(gs[n, g]))
            assert abs(Fraction(float(got[m, n])) - tot * Fraction(float(sw[n]))) <= abs(tot) * Fraction(1, 2 ** 50)


def test_linear_unit_scale_route():
    """With every scale 1 the symmetric epilogue returns the integer product itself."""
    rng = np.random.default_rng(11)
    qa = rng.integers(-7, 8, (4, 128))
    qb = rng.integers(-7, 8, (3, 128))
    acc = O.int_gemm(qa, qb)
    y = O.epilogue_sym_f32(acc, np.ones(4, np.float32), np.ones(3, np.float32))
    assert np.array_equal(y, (qa @ qb.T).astype(np.float32))


# ---------------------------------------------------------------- statistics
def _mixture_kurtosis(var):
    """Pearson kurtosis of a zero-mean Gaussian scale mixture with per-element variances `var`."""
    var = np.asarray(var, np.float64)
    return 3.0 * np.mean(var ** 2) / np.mean(var) ** 2


def test_kurtosis_gaussian_is_three():
    v = np.random.default_rng(12).standard_normal(4_000_000)
    assert abs(O.kurtosis(v) - 3.0) < 4 * math.sqrt(24 / v.size)


def test_kurtosis_qproj_before_and_after():
    """[ROT] "A rotation changes nothing": heavy tails before, near 3 after a full-width rotation."""
    d = WL.qproj(M=2048, with_w=False)
    x = d["X"].astype(np.float64)
    var_cols = np.ones(4096)
    var_cols[d["outlier_cols"]] = 30.0 ** 2
    before = _mixture_kurtosis(var_cols)
    assert abs(O.kurtosis(x) / before - 1) < 0.10          # ~2.5% sampling s.d. from 16k outlier draws
    full = O.kurtosis(O.rotate_normalized(x, 4096))
    assert abs(full - 3.0) < 0.05
    blk = O.kurtosis(O.rotate_normalized(x, 128))
    assert abs(blk / _mixture_kurtosis(var_cols.reshape(32, 128).mean(axis=1)) - 1) < 0.03


def test_kurtosis_downproj_blocks():
    """Token-varying spikes: per-128-block variance is (127 + 40^2)/128 where the spike sits, else 1."""
    d = WL.downproj(M=1024, with_w=False)
    y = O.rotate_normalized(d["X"], 128)
    nb = 14336 // 128
    var_blocks = np.concatenate([np.full(nb - 1, 1.0), [(127 + 1600.0) / 128]])
    assert abs(O.kurtosis(y) / _mixture_kurtosis(var_blocks) - 1) < 0.03


def test_kurtosis_kv_heads():
    d = WL.kv(B=1, H=4, S=1024)
    y = O.rotate_normalized(d["KV"].reshape(-1, 128), 128)
    assert abs(O.kurtosis(y) - 3.0) < 0.05
    assert O.kurtosis(d["KV"]) > 20


@pytest.mark.parametrize("cfg", ["tiny", "qproj", "downproj"])
def test_rotation_lowers_int4_product_error(cfg):
    """[ROT] "What it buys in 4 bits": INT4 per-token / per-channel product
    error is lower with the rotation than without (direction only)."""
    if cfg == "tiny":
        d = WL.tiny()
        x, w = d["X"], d["W"]
        blocks = [128]
    elif cfg == "qproj":
        d = WL.qproj(M=128)
        x, w = d["X"], d["W"][:512]
        blocks = [128, 4096]
    else:
        d = WL.downproj(M=128)
        x, w = d["X"], d["W"][:256]
        blocks = [128]
    px = O.quant_sym_rows(x.astype(np.float64), 1)
    pw = O.quant_sym_rows(w.astype(np.float64), 1)
    e_plain = O.product_error(x, w, O.dequant_sym_rows(px["codes"], px["scale"]),
                              O.dequant_sym_rows(pw["codes"], pw["scale"]))
    for b in blocks:
        r = O.w4a4_linear(x, w, b)
        e_rot = O.product_error(x, w, O.dequant_sym_rows(r["act"]["codes"], r["act"]["scale"]),
                                O.dequant_sym_rows(r["wq"]["codes"], r["wq"]["scale"]))
        assert e_rot < e_plain, (b, e_rot, e_plain)
        # the float64 product of the rotated, dequantized operands is the same Y as the oracle's
        ref = O.epilogue_sym_f64(r["acc"], r["act"]["scale"], r["wq"]["scale"])
        assert np.allclose(r["y"], ref, rtol=1e-12, atol=0)
    assert O.outlier_ratio(O.rotate_normalized(x, blocks[-1])) < O.outlier_ratio(x)


def test_asym_linear_matches_group_products():
    d = WL.gateup(M=8, N=64)
    r = O.w4a4_linear(d["X"], d["W"], 128, mode="asym")
    a, wq = r["act"], r["wq"]
    Ag = O.int_gemm_groups(a["codes"], a["zp"], wq["codes"])
    y = (Ag * a["scale"].astype(np.float64)[:, None, :]).sum(axis=2) * wq["scale"].astype(np.float64)[None, :]
    assert np.allclose(r["y"], y, rtol=1e-12, atol=1e-12)
    xq = O.dequant_asym_groups(a["codes"], a["scale"], a["zp"])
    wh = O.dequant_sym_rows(wq["codes"], wq["scale"])
    assert np.allclose(r["y"], xq @ wh.T, rtol=1e-10, atol=1e-10)


def test_kv_oracle_shapes_and_dequant():
    d = WL.kv(B=1, H=2, S=16)
    r = O.kv_rotate_quant(d["KV"], 128)
    assert r["packed"].shape == (1, 2, 16, 64) and r["scale"].shape == (1, 2, 16)
    y = O.rotate_normalized(d["KV"].reshape(-1, 128), 128)
    yh = O.dequant_asym_groups(r["codes"], r["scale"].reshape(-1, 1), r["zp"].reshape(-1, 1))
    assert np.all(np.abs(y - yh) <= 0.5 * r["scale"].reshape(-1, 1) * (1 + 1e-5))


# ---------------------------------------------------------------- randomized Hadamard (diag(d) H)
def test_signed_rotation_worked_example():
    """Hand-computed: d = (1, -1, 1, 1), x = (1, 2, 3, 4): d*x = (1, -2, 3, 4) and
    H4 (d*x) = (1-2+3+4, 1+2+3-4, 1-2-3-4, 1+2-3+4) = (6, 2, -8, 4)."""
    z = O.rotate(np.array([[1.0, 2.0, 3.0, 4.0]]), 4, signs=np.array([1.0, -1.0, 1.0, 1.0]))
    assert z.tolist() == [[6.0, 2.0, -8.0, 4.0]]


def test_all_plus_signs_is_the_plain_rotation():
    x = WL.small_random(11, 5, 512)
    for block in (128, 512):
        assert np.array_equal(O.rotate(x, block, signs=np.ones(512)), O.rotate(x, block))


@pytest.mark.parametrize("n", [2, 8, 64, 256])
def test_signed_hadamard_orthogonal(n):
    """(diag(d) H)^T (diag(d) H) = H^T diag(d)^2 H = n I, exactly in integers."""
    d = WL.hadamard_signs(n, seed=n).astype(np.int64)
    m = d[:, None] * O.hadamard(n)
    assert np.array_equal(m.T @ m, n * np.eye(n, dtype=np.int64))


@pytest.mark.parametrize("block", [128, 1024])
def test_signed_invariance_and_mismatch(block):
    """Same d on both sides: X W^T is unchanged to float64 rounding; different d
    on the two sides: the product is destroyed (the diagonal must be shared)."""
    x = WL.small_random(21, 64, 1024, outlier_cols=(5,), mult=30.0).astype(np.float64)
    w = WL.small_random(22, 48, 1024, std=0.02).astype(np.float64)
    d = WL.hadamard_signs(1024, seed=3)
    ref = x @ w.T
    same = O.rotate_normalized(x, block, d) @ O.rotate_normalized(w, block, d).T
    assert np.linalg.norm(same - ref) / np.linalg.norm(ref) < 1e-10
    other = O.rotate_normalized(x, block, d) @ O.rotate_normalized(w, block, WL.hadamard_signs(1024, seed=4)).T
    assert np.linalg.norm(other - ref) / np.linalg.norm(ref) > 0.5


@pytest.mark.parametrize("n,j", [(128, 5), (128, 77), (512, 300)])
def test_signed_outlier_codes_closed_form(n, j):
    """x = M e_j: d*x = M d_j e_j, so z = M d_j h_j and the symmetric codes are
    7 d_j (-1)^popcount(i & j) with scale M / (7 sqrt(n)) -- exactly."""
    m = 96.0
    x = np.zeros((1, n))
    x[0, j] = m
    d = WL.hadamard_signs(n, seed=j)
    expect = np.array([7 * int(d[j]) * (-1) ** bin(i & j).count("1") for i in range(n)])
    for decide in ("f64", "f32"):
        q = O.rotate_quant_act(x, n, "sym", signs=d, decide=decide)
        assert np.array_equal(q["codes"][0], expect)
    assert q["scale"][0] == np.float32(np.float32(m) / np.float32(7.0 * math.sqrt(n)))
    assert math.isclose(O.rotate_quant_act(x, n, "sym", signs=d)["scale"][0], m / (7.0 * math.sqrt(n)),
                        rel_tol=4e-16)


def test_signed_rotation_lowers_int4_product_error():
    """The randomized rotation keeps the page's effect: the INT4 product error
    with diag(d) H is far below the unrotated one (q_proj-like outliers)."""
    d = WL.qproj(M=256, with_w=False)
    x = d["X"].astype(np.float64)
    w = WL.qproj_weight()[:256].astype(np.float64)
    s = WL.hadamard_signs(4096, seed=1)
    plain_q = O.quant_sym_rows(x, 1)
    plain_w = O.quant_sym_rows(w, 1)
    e_plain = O.product_error(x, w, O.dequant_sym_rows(plain_q["codes"], plain_q["scale"]),
                              O.dequant_sym_rows(plain_w["codes"], plain_w["scale"]))
    lin = O.w4a4_linear(x, w, 128, "sym", signs=s)
    ref = x @ w.T
    e_rot = np.linalg.norm(lin["y"] - ref) / np.linalg.norm(ref)
    assert e_rot < 0.5 * e_plain


# ---------------------------------------------------------------- decode attention over the INT4 KV cache
def test_attention_decode_brute_force():
    """Python loops with math.exp on a tiny case."""
    rng = np.random.default_rng(1)
    B, H, S, D = 1, 2, 5, 4
    q = rng.standard_normal((B, H, D))
    k = rng.standard_normal((B, H, S, D))
    v = rng.standard_normal((B, H, S, D))
    o = O.attention_decode_f64(q, k, v, 0.7)
    for h in range(H):
        sc = [0.7 * sum(q[0, h, d] * k[0, h, t, d] for d in range(D)) for t in range(S)]
        mx = max(sc)
        e = [math.exp(x - mx) for x in sc]
        z = sum(e)
        for d in range(D):
            want = sum(e[t] / z * v[0, h, t, d] for t in range(S))
            assert abs(o[0, h, d] - want) < 1e-12


def test_attention_decode_closed_forms():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((1, 1, 9, 8))
    v = rng.standard_normal((1, 1, 9, 8))
    # q = 0: every score equal -> the mean of v
    assert np.allclose(O.attention_decode_f64(np.zeros((1, 1, 8)), k, v, 1.0), v.mean(axis=2), atol=1e-14)
    # one key far above the rest -> that key's value
    q = np.zeros((1, 1, 8))
    q[0, 0, 0] = 1.0
    k2 = np.zeros_like(k)
    k2[0, 0, 4, 0] = 1000.0
    assert np.allclose(O.attention_decode_f64(q, k2, v, 1.0), v[:, :, 4], atol=1e-12)


@pytest.mark.parametrize("with_signs", [False, True])
def test_rotated_attention_invariance(with_signs):
    """softmax((qQ)(kQ)^T) (vQ) Q^T = softmax(q k^T) v for orthogonal Q = diag(d) H / sqrt(128)."""
    rng = np.random.default_rng(3)
    B, H, S, D = 2, 3, 40, 128
    q = rng.standard_normal((B, H, D))
    k = rng.standard_normal((B, H, S, D))
    v = rng.standard_normal((B, H, S, D))
    d = WL.hadamard_signs(D, seed=9) if with_signs else None
    rot = lambda a: O.rotate_normalized(a.reshape(-1, D), D, d).reshape(a.shape)   # noqa: E731
    o_rot = O.attention_decode_f64(rot(q), rot(k), rot(v), 0.125)
    back = O.apply_signs(O.rotate_normalized(o_rot.reshape(-1, D), D), d).reshape(B, H, D)
    assert np.max(np.abs(back - O.attention_decode_f64(q, k, v, 0.125))) < 1e-12


@pytest.mark.parametrize("with_signs", [False, True])
def test_kv4_attention_matches_original_domain(with_signs):
    """kv4_attention_decode (scores and weighted sum in the rotated domain,
    output rotated back) equals plain attention over the dequantized K and V
    rotated back to the original domain first: checks the rotation bookkeeping."""
    kvd = WL.kv(B=1, H=2, S=64)
    kv = kvd["KV"]
    vv = WL.kv(B=1, H=2, S=64)["KV"][:, :, ::-1].copy()
    q = WL.small_random(4, 2, 128).reshape(1, 2, 128)
    D = 128
    d = WL.hadamard_signs(D, seed=1) if with_signs else None
    kq = O.kv_rotate_quant(kv, signs=d)
    vq = O.kv_rotate_quant(vv, signs=d)
    o = O.kv4_attention_decode(q, kq["packed"], kq["scale"], kq["zp"], vq["packed"], vq["scale"], vq["zp"],
                               1 / math.sqrt(D), signs=d)

    def unrot(qd, shape):
        u = O.unpack_nibbles(qd["packed"].reshape(-1, D // 2), signed=False)
        yhat = O.dequant_asym_groups(u, qd["scale"].reshape(-1, 1), qd["zp"].reshape(-1, 1), D)
        return O.apply_signs(O.rotate_normalized(yhat, D), d).reshape(shape)

    want = O.attention_decode_f64(q, unrot(kq, kv.shape), unrot(vq, vv.shape), 1 / math.sqrt(D))
    assert np.max(np.abs(o - want)) < 1e-10
    # the rotation helps the 4-bit cache: the same asymmetric quantizer on the
    # unrotated head vectors gives a larger attention error (outlier dims x20)
    exact = O.attention_decode_f64(q, kv, vv, 1 / math.sqrt(D))

    def plain(x):
        g = O.quant_asym_groups(x.reshape(-1, D).astype(np.float64), 1, D)
        return O.dequant_asym_groups(g["codes"], g["scale"], g["zp"], D).reshape(x.shape)

    e_rot = np.linalg.norm(o - exact) / np.linalg.norm(exact)
    e_plain = np.linalg.norm(O.attention_decode_f64(q, plain(kv), plain(vv), 1 / math.sqrt(D)) - exact) \
        / np.linalg.norm(exact)
    assert e_rot < e_plain


# ---------------------------------------------------------------- MXFP4 (E2M1 + power-of-two scale per 32)
def _e2m1_from_bits(c):
    """E2M1 from its bit fields: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0;
    exponent 0 is subnormal (0.5 m)."""
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


def test_e2m1_decode_matches_bit_fields():
    for c in range(16):
        assert O.e2m1_value([c])[0] == float(_e2m1_from_bits(c))


def test_e2m1_round_brute_force():
    """Every multiple of 1/8 in [-8, 8]: nearest representable value, ties to the
    even mantissa, saturation at +-6, no negative zero."""
    values = [Fraction(i, 8) for i in range(-64, 65)]
    codes = O.e2m1_round([float(v) for v in values])
    grid = [(c, _e2m1_from_bits(c)) for c in range(8)]
    for v, got in zip(values, codes):
        a = min(abs(v), Fraction(6))
        best = min(abs(a - g) for _, g in grid)
        near = [c for c, g in grid if abs(a - g) == best]
        c = near[0] if len(near) == 1 else [c for c in near if c % 2 == 0][0]
        want = c + (8 if v < 0 and c > 0 else 0)
        assert got == want, (v, got, want)


def test_mx_scale_worked_examples():
    """Hand-worked blocks: amax 6 -> e = 0 (6 exact); amax 3 -> e = -1 (3 -> 6, 1 -> 2);
    amax 0.3 -> floor(log2 0.3) = -2, e = -4, 0.3 * 16 = 4.8 -> nearest 4 (code 6);
    amax 7 -> e = 0 and 7 saturates to 6; a zero block -> byte 0, codes 0."""
    y = np.zeros((5, 32), np.float32)
    y[0, 0], y[0, 1] = 6.0, -0.5
    y[1, 0], y[1, 1] = 3.0, 1.0
    y[2, 0] = 0.3
    y[3, 0] = 7.0
    q = O.mx_quant_rows(y)
    assert list(q["scale_e"][:, 0]) == [0, -1, -4, 0, -127]
    assert list(q["scale_byte"][:, 0]) == [127, 126, 123, 127, 0]
    assert (q["codes"][0, 0], q["codes"][0, 1]) == (7, 9)
    assert (q["codes"][1, 0], q["codes"][1, 1]) == (7, 4)
    assert q["codes"][2, 0] == 6 and q["codes"][3, 0] == 7
    assert np.all(q["codes"][4] == 0)


def test_mx_quant_invariants():
    y = WL.small_random(31, 64, 256, outlier_cols=(7,), mult=50.0).astype(np.float32)
    q = O.mx_quant_rows(y)
    deq = O.mx_dequant_rows(q["codes"], q["scale_e"])
    yb = y.astype(np.float64).reshape(64, 8, 32)
    scale = np.exp2(q["scale_e"].astype(np.float64))[..., None]
    t = np.abs(yb) / scale
    # up to 6 * 2^e the error is at most half the local grid step; above it
    # (the block maximum lands in [4, 8), so values in (6, 8) exist) the value
    # saturates to +-6 * 2^e
    deq = deq.reshape(64, 8, 32)
    step = np.where(t < 2, 0.5, np.where(t < 4, 1.0, 2.0))
    inside = t <= 6
    assert np.all(np.abs(deq - yb)[inside] <= (step * scale / 2)[inside])
    assert np.all(np.abs(deq)[~inside] == (6 * scale * np.ones_like(t))[~inside])
    amax_t = t.max(axis=-1)
    assert np.all((amax_t >= 4) & (amax_t < 8))


def test_mx_gemm_brute_force():
    rng = np.random.default_rng(5)
    ca = rng.integers(0, 16, (3, 64))
    cb = rng.integers(0, 16, (2, 64))
    ea = rng.integers(-6, 6, (3, 2))
    eb = rng.integers(-6, 6, (2, 2))
    y = O.mx_gemm_f64(ca, ea, cb, eb)
    for m in range(3):
        for n in range(2):
            acc = Fraction(0)
            for k in range(64):
                j = k // 32
                acc += _e2m1_from_bits(int(ca[m, k])) * _e2m1_from_bits(int(cb[n, k])) \
                    * Fraction(2) ** int(ea[m, j] + eb[n, j])
            assert y[m, n] == float(acc)


def test_rotation_lowers_mxfp4_product_error():
    """[ROT] "Gotchas": rotations help MXFP4 -- q_proj-like fixed outlier channels."""
    d = WL.qproj(M=256, with_w=False)
    x = d["X"].astype(np.float64)
    w = WL.qproj_weight()[:256].astype(np.float64)
    ref = x @ w.T

    def err(xq, wq):
        return np.linalg.norm(xq @ wq.T - ref) / np.linalg.norm(ref)

    plain = err(O.mx_dequant_rows(**{k: v for k, v in O.mx_quant_rows(x.astype(np.float32)).items()
                                     if k in ("codes", "scale_e")}),
                O.mx_dequant_rows(**{k: v for k, v in O.mx_quant_rows(w.astype(np.float32)).items()
                                     if k in ("codes", "scale_e")}))
    for block in (128, 4096):
        qa, qw = O.rotate_mx_quant(x, block), O.rotate_mx_quant(w, block)
        rot = err(O.mx_dequant_rows(qa["codes"], qa["scale_e"]), O.mx_dequant_rows(qw["codes"], qw["scale_e"]))
        assert rot < plain, (block, rot, plain)
