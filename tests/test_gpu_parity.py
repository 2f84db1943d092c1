"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every input comes from `workloads`; every expected value from `oracle`.
Rules (tests/parity.py): codes may differ only at .5 ties of the oracle's
pre-rounding value (<= 1e-4 of elements, one level), scales agree to 1e-6
relative, packed bytes agree wherever both codes agree, integer products are
exact, dequantized outputs agree to 1e-3 relative Frobenius error; inputs of
the exact-arithmetic class must match bit for bit.
"""
import numpy as np
import pytest

import oracle as O
import workloads as WL
from parity import Y_RTOL_FRO, check_asym, check_gsum, check_sym, rel_fro

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


def gpu_act(x, block, mode="sym"):
    c, s, z = R.rotate_quant_act(dev(x), had_block=block, act_mode=mode)
    return host(c), host(s), (None if z is None else host(z))


# ---------------------------------------------------------------- rotate + quantize (activations)
@pytest.mark.parametrize("cfg,block", [("tiny", 128), ("qproj", 128), ("qproj", 4096),
                                       ("downproj", 128), ("decode1", 128), ("decode4", 128),
                                       ("decode16", 128)])
def test_rotate_quant_act_configs(cfg, block):
    if cfg == "tiny":
        x = WL.tiny()["X"]
    elif cfg == "qproj":
        x = WL.qproj(with_w=False)["X"]
    elif cfg == "downproj":
        x = WL.downproj(with_w=False)["X"]
    else:
        x = WL.decode(int(cfg[6:]), with_w=False)["X"]
    c, s, _ = gpu_act(x, block)
    ref = O.quant_sym_rows(O.rotate(x, block), block)
    st = check_sym(c, s, ref)
    print(cfg, block, st)


@pytest.mark.parametrize("K", [128, 256, 384, 640, 1152, 2048, 2176, 4096, 8192, 14336, 16384])
@pytest.mark.parametrize("M", [1, 37, 300])
def test_rotate_quant_act_shapes(M, K):
    x = WL.small_random(M * 7 + K, M, K, outlier_cols=[K // 3, K - 1], mult=35.0)
    c, s, _ = gpu_act(x, 128)
    check_sym(c, s, O.quant_sym_rows(O.rotate(x, 128), 128))
    if K & (K - 1) == 0:
        c, s, _ = gpu_act(x, "full")
        check_sym(c, s, O.quant_sym_rows(O.rotate(x, K), K))


@pytest.mark.parametrize("K,block", [(128, 128), (1024, 128), (4096, 128), (4096, 4096),
                                     (8192, 8192), (2048, 2048), (14336, 128)])
def test_rotate_quant_exact_class_bitexact(K, block):
    """Integer inputs <= 2048 and blocks <= 8192: the fp32 transform is exact,
    so codes, scales and bytes must equal the oracle's bit for bit."""
    x = WL.exact_class(K + block, 64, K, lim=2048, outlier_cols=[5, K // 2])
    c, s, _ = gpu_act(x, "full" if block == K and K > 128 else 128)
    z = O.rotate(x, block)
    check_sym(c, s, O.quant_sym_rows(z, block, "f32"), exact=True)
    check_sym(c, s, O.quant_sym_rows(z, block))


def test_rotate_quant_edge_rows():
    K = 512
    x = np.zeros((6, K), np.float16)
    x[1] = 3.0                                  # constant row
    x[2, 17] = -60000.0                         # one-hot, near the fp16 maximum
    x[3] = np.float16(6e-8)                     # fp16 subnormals
    x[4, ::2] = 1.0
    x[4, 1::2] = -1.0
    x[5] = WL.small_random(9, 1, K)[0]
    for block in (128, "full"):
        b = 128 if block == 128 else K
        c, s, _ = gpu_act(x, block)
        ref = O.quant_sym_rows(O.rotate(x, b), b)
        check_sym(c, s, ref)
        assert s[0] == 0 and np.all(c[0] == 0)


def test_rotate_quant_row_stride_and_determinism():
    x = WL.small_random(11, 50, 1024 + 64, outlier_cols=[3], mult=40.0)
    xt = dev(x)[:, :1024]                        # ldx = 1088 > K
    c1, s1, _ = R.rotate_quant_act(xt, 128)
    c2, s2, _ = R.rotate_quant_act(dev(np.ascontiguousarray(x[:, :1024])), 128)
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    c3, s3, _ = R.rotate_quant_act(xt, 128)
    assert torch.equal(c1, c3) and torch.equal(s1, s3)
    check_sym(host(c1), host(s1), O.quant_sym_rows(O.rotate(x[:, :1024], 128), 128))


def test_rotate_quant_empty():
    x = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    c, s, _ = R.rotate_quant_act(x, 128)
    assert c.shape == (0, 128) and s.shape == (0,)


def test_empty_batches_are_no_ops():
    """Zero rows (M = 0, N = 0, S = 0, B = 0) return OK and launch nothing,
    symmetric and asymmetric, through every quantize and GEMM entry point."""
    c, s, z = R.rotate_quant_act(torch.empty((0, 256), dtype=torch.float16, device="cuda"), 128, act_mode="asym")
    assert c.shape == (0, 128) and s.shape == (0, 2) and z.shape == (0, 2)
    wc, ws, wg = R.quant_weight_offline(torch.empty((0, 256), dtype=torch.float16, device="cuda"), 128)
    assert wc.shape == (0, 128) and ws.shape == (0,) and wg.shape == (0, 2)
    for B, H, S in ((0, 4, 16), (2, 0, 16), (2, 4, 0)):
        kc, ks, kz = R.kv_rotate_quant4(torch.empty((B, H, S, 128), dtype=torch.float16, device="cuda"))
        assert kc.shape == (B, H, S, 64) and ks.shape == (B, H, S) and kz.shape == (B, H, S)
    w = torch.zeros((8, 128), dtype=torch.uint8, device="cuda")
    one = torch.ones((8,), dtype=torch.float32, device="cuda")
    xc = torch.empty((0, 128), dtype=torch.uint8, device="cuda")
    y = R.w4a4_gemm(xc, torch.empty((0,), dtype=torch.float32, device="cuda"), None, w, one)
    assert y.shape == (0, 8)
    y = R.w4a4_gemm(xc, torch.empty((0, 2), dtype=torch.float32, device="cuda"),
                    torch.empty((0, 2), dtype=torch.uint8, device="cuda"), w, one, act_mode="asym")
    assert y.shape == (0, 8)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- asymmetric activations and KV
@pytest.mark.parametrize("M,K", [(256, 8192), (1, 128), (37, 384), (300, 2176)])
def test_rotate_quant_asym(M, K):
    if K == 8192:
        x = WL.gateup(M=M, with_w=False)["X"]
    else:
        x = WL.small_random(M + K, M, K, outlier_cols=[1, K - 7], mult=30.0)
    c, s, z = gpu_act(x, 128, "asym")
    st = check_asym(c, s, z, O.quant_asym_groups(O.rotate(x, 128), 128))
    print(M, K, st)


def test_rotate_quant_asym_exact_class():
    x = WL.exact_class(3, 128, 1024, lim=2048, outlier_cols=[0, 700])
    x[5] = 0
    x[6, :] = 7                                   # all rotated mass at index 0 of each block
    x[7, :128] = np.arange(128) - 64              # a group with both signs
    c, s, z = gpu_act(x, 128, "asym")
    zr = O.rotate(x, 128)
    check_asym(c, s, z, O.quant_asym_groups(zr, 128, mode="f32"), exact=True)
    check_asym(c, s, z, O.quant_asym_groups(zr, 128))


def test_kv_rotate_quant4_small_and_strided():
    d = WL.kv(B=2, H=4, S=100)
    kv = d["KV"]
    c, s, z = R.kv_rotate_quant4(dev(kv))
    ref = O.kv_rotate_quant(kv)
    flat = dict(ref, scale=ref["scale"].reshape(-1, 1), zp=ref["zp"].reshape(-1, 1))
    check_asym(host(c).reshape(-1, 64), host(s).reshape(-1, 1), host(z).reshape(-1, 1), flat)
    # a [B, S, H, D] buffer viewed as [B, H, S, D]: non-dense strides
    bshd = dev(np.ascontiguousarray(kv.transpose(0, 2, 1, 3)))
    c2, s2, z2 = R.kv_rotate_quant4(bshd.permute(0, 2, 1, 3))
    assert torch.equal(c, c2) and torch.equal(s, s2) and torch.equal(z, z2)


def test_kv_rotate_quant4_full_config_all_heads():
    """The whole KV config, 8 x 32 x 4096 head vectors of 128: every (batch,
    head) compared with the oracle, one batch row (4 Mi elements) at a time."""
    d = WL.kv()
    kv = d["KV"]
    c, s, z = R.kv_rotate_quant4(dev(kv))
    c, s, z = host(c), host(s), host(z)
    flips = zp_flips = 0
    for b in range(kv.shape[0]):
        ref = O.kv_rotate_quant(kv[b][None])
        flat = dict(ref, scale=ref["scale"].reshape(-1, 1), zp=ref["zp"].reshape(-1, 1))
        st = check_asym(c[b].reshape(-1, 64), s[b].reshape(-1, 1), z[b].reshape(-1, 1), flat)
        flips += st["flips"]
        zp_flips += st["zp_flips"]
    print("kv all heads: level flips", flips, "zero-point flips", zp_flips, "of", kv.size)


# ---------------------------------------------------------------- offline weights
@pytest.mark.parametrize("block", [128, 4096])
def test_quant_weight_offline(block):
    w = WL.qproj_weight()
    c, s, g = R.quant_weight_offline(dev(w), had_block=block if block == 128 else "full")
    c, s, g = host(c), host(s), host(g)
    ref = O.quant_weight_offline(w, block)
    check_sym(c, s, ref)
    check_gsum(g, c, ref)


# ---------------------------------------------------------------- GEMM on identical codes
def _rand_codes(seed, rows, K, lo=-7, hi=7):
    return np.random.default_rng(seed).integers(lo, hi + 1, (rows, K))


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (4, 100, 256), (16, 4096, 4096), (17, 257, 1152),
                                   (128, 128, 128), (300, 200, 384), (2048, 512, 4096),
                                   (129, 130, 14336), (513, 100, 640), (4096, 4096, 256),
                                   (2048, 4096, 128)])
def test_gemm_same_codes_sym_bitexact(M, N, K):
    qa = _rand_codes(M * N + K, M, K)
    qb = _rand_codes(M + N * K, N, K)
    rng = np.random.default_rng(K)
    sx = (rng.random(M) * 2 + 0.01).astype(np.float32)
    sw = (rng.random(N) * 0.01 + 1e-4).astype(np.float32)
    y = R.w4a4_gemm(dev(O.pack_nibbles(qa)), dev(sx), None, dev(O.pack_nibbles(qb)), dev(sw))
    want = O.epilogue_sym_f32(O.int_gemm(qa, qb), sx, sw)
    assert np.array_equal(host(y), want)


@pytest.mark.parametrize("M", [1, 16, 200])
def test_gemm_unit_scales_give_exact_integers(M):
    K, N = 14336, 64
    qa = np.full((M, K), -7)
    qa[:, ::3] = 7
    qb = _rand_codes(5, N, K)
    qb[0] = -7
    ones_m, ones_n = np.ones(M, np.float32), np.ones(N, np.float32)
    y = host(R.w4a4_gemm(dev(O.pack_nibbles(qa)), dev(ones_m), None, dev(O.pack_nibbles(qb)), dev(ones_n)))
    acc = O.int_gemm(qa, qb)
    assert np.array_equal(y, acc.astype(np.float32)) and np.abs(acc).max() < 2 ** 24


@pytest.mark.parametrize("M,N,K", [(5, 64, 128), (128, 128, 1024), (300, 129, 8192), (16, 16, 256)])
def test_gemm_same_codes_asym(M, N, K):
    rng = np.random.default_rng(M + N + K)
    G = K // 128
    u = rng.integers(0, 16, (M, K))
    zp = rng.integers(0, 16, (M, G))
    qw = _rand_codes(N, N, K)
    sx = (rng.random((M, G)) + 0.05).astype(np.float32)
    sw = (rng.random(N) * 0.01 + 1e-4).astype(np.float32)
    y = R.w4a4_gemm(dev(O.pack_nibbles(u)), dev(sx), dev(zp.astype(np.uint8)), dev(O.pack_nibbles(qw)),
                    dev(sw), act_mode="asym")
    want = O.gemm_asym_f64(u, zp, sx, qw, sw)
    assert rel_fro(host(y), want) < 1e-6


def test_gemm_output_stride():
    M, N, K = 40, 72, 256
    qa, qb = _rand_codes(1, M, K), _rand_codes(2, N, K)
    sx, sw = np.ones(M, np.float32), np.ones(N, np.float32)
    out = torch.full((M, N + 24), -1.0, device="cuda")[:, :N]
    R.w4a4_gemm(dev(O.pack_nibbles(qa)), dev(sx), None, dev(O.pack_nibbles(qb)), dev(sw), out=out)
    full = host(out.as_strided((M, N + 24), (N + 24, 1)))
    assert np.array_equal(full[:, :N], O.int_gemm(qa, qb).astype(np.float32))
    assert np.all(full[:, N:] == -1.0)



@pytest.mark.parametrize("M,N,K,pad", [(40, 72, 256, 3), (600, 300, 512, 5), (2048, 4096, 256, 1),
                                       (2048, 4100, 256, 0), (513, 4096, 384, 2)])
def test_gemm_output_stride_unaligned(M, N, K, pad):
    """Row strides that are not a multiple of 4 floats, and ragged N, take the
    scalar stores of the output epilogue (64-row and 256-row tilings); the
    values still match the oracle's fp32 epilogue bit for bit and nothing past
    column N is written."""
    qa, qb = _rand_codes(M + 7, M, K), _rand_codes(N + 11, N, K)
    rng = np.random.default_rng(M * N + pad)
    sx = (rng.random(M) * 2 + 0.01).astype(np.float32)
    sw = (rng.random(N) * 0.01 + 1e-4).astype(np.float32)
    buf = torch.full((M, N + pad), -1.0, device="cuda")
    R.w4a4_gemm(dev(O.pack_nibbles(qa)), dev(sx), None, dev(O.pack_nibbles(qb)), dev(sw), out=buf[:, :N])
    full = host(buf)
    assert np.array_equal(full[:, :N], O.epilogue_sym_f32(O.int_gemm(qa, qb), sx, sw))
    assert np.all(full[:, N:] == -1.0)


@pytest.mark.parametrize("M,N,K,pad", [(130, 260, 256, 3), (300, 129, 384, 1)])
def test_gemm_asym_output_stride_unaligned(M, N, K, pad):
    """Asymmetric kernel, unaligned row stride: the same values as a
    contiguous output (only the store addresses differ), within the oracle's
    tolerance, and nothing past column N is written."""
    rng = np.random.default_rng(M + N + K + pad)
    G = K // 128
    u = rng.integers(0, 16, (M, K))
    zp = rng.integers(0, 16, (M, G))
    qw = _rand_codes(N + 5, N, K)
    sx = (rng.random((M, G)) + 0.05).astype(np.float32)
    sw = (rng.random(N) * 0.01 + 1e-4).astype(np.float32)
    args = (dev(O.pack_nibbles(u)), dev(sx), dev(zp.astype(np.uint8)), dev(O.pack_nibbles(qw)), dev(sw))
    y = host(R.w4a4_gemm(*args, act_mode="asym"))
    buf = torch.full((M, N + pad), -1.0, device="cuda")
    R.w4a4_gemm(*args, act_mode="asym", out=buf[:, :N])
    full = host(buf)
    assert np.array_equal(full[:, :N], y)
    assert np.all(full[:, N:] == -1.0)
    assert rel_fro(y, O.gemm_asym_f64(u, zp, sx, qw, sw)) < 1e-6

# ---------------------------------------------------------------- end to end
def _e2e(x, w, block, mode="sym"):
    hb = block if block == 128 else "full"
    xc, xs, xz = R.rotate_quant_act(dev(x), hb, mode)
    wc, ws, wg = R.quant_weight_offline(dev(w), hb)
    y = R.w4a4_gemm(xc, xs, xz, wc, ws, wg, act_mode=mode)
    return host(y)


@pytest.mark.parametrize("cfg,block", [("tiny", 128), ("qproj", 128), ("qproj", 4096),
                                       ("decode1", 128), ("decode4", 128), ("decode16", 128)])
def test_linear_end_to_end(cfg, block):
    if cfg == "tiny":
        d = WL.tiny()
    elif cfg == "qproj":
        d = WL.qproj()
    else:
        d = WL.decode(int(cfg[6:]))
    y = _e2e(d["X"], d["W"], block)
    ref = O.w4a4_linear(d["X"], d["W"], block)
    err = rel_fro(y, ref["y"])
    print(cfg, block, "rel_fro", err)
    assert err <= Y_RTOL_FRO


def test_linear_downproj_full_size():
    """The whole down_proj layer, 4096 x 4096 outputs over K = 14336, against
    the oracle's whole pipeline (its integer product is exact in float64)."""
    d = WL.downproj()
    y = _e2e(d["X"], d["W"], 128)
    ref = O.w4a4_linear(d["X"], d["W"], 128)
    err = rel_fro(y, ref["y"])
    print("downproj rel_fro", err)
    assert err <= Y_RTOL_FRO


def test_linear_gateup_asym_full_size_512_rows():
    """gate/up at full size on the GPU (8192 x 28672 over K = 8192); the
    oracle quantizes every weight row and computes 512 seeded activation rows
    against all 28672 output columns (rows are independent: each output row
    depends on its own activation row and every weight row)."""
    d = WL.gateup()
    y = _e2e(d["X"], d["W"], 128, mode="asym")
    rows = np.sort(np.random.default_rng(4).choice(8192, 512, replace=False))
    ref = O.w4a4_linear(d["X"][rows], d["W"], 128, mode="asym")
    err = rel_fro(y[rows], ref["y"])
    print("gateup rel_fro", err)
    assert err <= Y_RTOL_FRO
