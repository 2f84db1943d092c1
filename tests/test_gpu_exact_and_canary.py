"""GPU parity at the headline GEMM shapes on identical codes, exact integer
products of the asymmetric kernel, and canary bytes after every output.

"Rotations for 4-Bit Activations: QuaRot, SpinQuant, and Friends", section
"A rotation changes nothing, and that is the point": on codes the layer is an
integer product, so with identical codes the int32 accumulators (and the
fp32 epilogue of the symmetric kernel) must equal the oracle's bit for bit.
SpinQuant page, "Activation scheme": per-group asymmetric activations; with
unit scales every group's integer sum and their fp32 total are exact
(|sum| <= 15 * 7 * K < 2^24), so the asymmetric kernel must return the
oracle's integers exactly, whatever the zero-points.
"""
import ctypes

import numpy as np
import pytest

import oracle as O
import workloads as WL
from parity import check_asym, check_gsum, check_mx, check_sym, rel_fro

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import rotation_w4a4_quantization_amd as R
    from rotation_w4a4_quantization_amd import _lib


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _codes(seed, rows, K, lo=-7, hi=7):
    return np.random.default_rng(seed).integers(lo, hi + 1, (rows, K))


# ---------------------------------------------------------------- symmetric, headline shapes
@pytest.mark.parametrize("M,N,K", [(2048, 4096, 4096), (4096, 4096, 14336), (2048, 4096, 1152),
                                   (4096, 4096, 4224)])
def test_gemm_same_codes_sym_bitexact_large(M, N, K):
    """The 256-row kernel's long K loop (32, 112, 9 and 33 K-steps: both
    parities of the LDS stage ring): bit-exact against the oracle's fp32
    epilogue of the exact integer product."""
    qa = _codes(M + K, M, K)
    qb = _codes(N * 3 + K, N, K)
    rng = np.random.default_rng(M ^ K)
    sx = (rng.random(M) * 2 + 0.01).astype(np.float32)
    sw = (rng.random(N) * 0.01 + 1e-4).astype(np.float32)
    y = host(R.w4a4_gemm(dev(O.pack_nibbles(qa)), dev(sx), None, dev(O.pack_nibbles(qb)), dev(sw)))
    want = O.epilogue_sym_f32(O.int_gemm(qa, qb), sx, sw)
    assert np.array_equal(y, want)


@pytest.mark.parametrize("M,N,K", [(640, 4096, 640), (1536, 4096, 128), (1000, 3000, 1408), (700, 5000, 384),
                                   (512, 4096, 256), (1536, 4096, 4096)])
def test_gemm_same_codes_sym_bitexact_small_grids(M, N, K):
    """Shapes with fewer than 256 tiles of 256 rows.  From 160 tiles of 128
    rows the 4-wave 32x32-block kernel runs (1, 3, 5, 11 and 32 K-steps,
    ragged M and N); 512 x 4096 (128 such tiles) takes the 64-row kernel.
    Bit-exact against the oracle's fp32 epilogue of the exact product."""
    qa = _codes(M + 5 * K, M, K)
    qb = _codes(N + 7 * K, N, K)
    rng = np.random.default_rng(M + N + K)
    sx = (rng.random(M) * 2 + 0.01).astype(np.float32)
    sw = (rng.random(N) * 0.01 + 1e-4).astype(np.float32)
    y = host(R.w4a4_gemm(dev(O.pack_nibbles(qa)), dev(sx), None, dev(O.pack_nibbles(qb)), dev(sw)))
    assert np.array_equal(y, O.epilogue_sym_f32(O.int_gemm(qa, qb), sx, sw))


# ---------------------------------------------------------------- asymmetric, exact integers
def _asym_case(M, N, K, seed, zp=None):
    rng = np.random.default_rng(seed)
    G = K // 128
    u = rng.integers(0, 16, (M, K))
    if zp is None:
        zp = rng.integers(0, 16, (M, G))
    qw = _codes(seed + 1, N, K)
    return u, zp, qw


@pytest.mark.parametrize("M,N,K", [(16, 64, 128), (300, 129, 8192), (2048, 4096, 1152), (2048, 4096, 1024),
                                   (513, 4096, 14336)])
def test_gemm_asym_unit_scales_exact_integers(M, N, K):
    """Unit scales: Y = sum over groups of (u - zp) . q_w, an integer below 2^24
    that fp32 holds exactly at every partial sum, so the GPU must return the
    oracle's integer product exactly.  (2048, 4096, *) runs the 256-row
    instance with 9 (odd) and 8 (even) groups; the others the 128-row one."""
    u, zp, qw = _asym_case(M, N, K, M * 7 + K)
    G = K // 128
    ones_g, ones_n = np.ones((M, G), np.float32), np.ones(N, np.float32)
    y = host(R.w4a4_gemm(dev(O.pack_nibbles(u)), dev(ones_g), dev(zp.astype(np.uint8)),
                         dev(O.pack_nibbles(qw)), dev(ones_n), act_mode="asym"))
    lv = u.reshape(M, G, 128) - zp[:, :, None]
    want = O.int_gemm(lv.reshape(M, K), qw)
    assert np.abs(want).max() < 2 ** 24
    assert np.array_equal(y, want.astype(np.float32))


def test_gemm_asym_every_zero_point_single_group():
    """K = 128 with each of the 16 zero-points on its own rows."""
    M, N, K = 64, 96, 128
    zp = (np.arange(M) % 16)[:, None]
    u, _, qw = _asym_case(M, N, K, 99, zp=zp)
    y = host(R.w4a4_gemm(dev(O.pack_nibbles(u)), dev(np.ones((M, 1), np.float32)), dev(zp.astype(np.uint8)),
                         dev(O.pack_nibbles(qw)), dev(np.ones(N, np.float32)), act_mode="asym"))
    assert np.array_equal(y, O.int_gemm(u - zp, qw).astype(np.float32))


@pytest.mark.parametrize("M,N,K", [(2048, 4096, 1152), (2048, 4096, 1024)])
def test_gemm_asym_same_codes_256_row_instance(M, N, K):
    """Random scales through the 256-row asymmetric instance (odd and even
    group counts): within 1e-6 of the oracle's float64 sum of group products."""
    u, zp, qw = _asym_case(M, N, K, M + 3 * K)
    rng = np.random.default_rng(K)
    sx = (rng.random((M, K // 128)) + 0.05).astype(np.float32)
    sw = (rng.random(N) * 0.01 + 1e-4).astype(np.float32)
    y = host(R.w4a4_gemm(dev(O.pack_nibbles(u)), dev(sx), dev(zp.astype(np.uint8)), dev(O.pack_nibbles(qw)),
                         dev(sw), act_mode="asym"))
    err = rel_fro(y, O.gemm_asym_f64(u, zp, sx, qw, sw))
    print(M, N, K, "rel_fro", err)
    assert err < 1e-6


@pytest.mark.parametrize("M,N,K", [(2000, 4000, 128), (2000, 4000, 256), (2000, 4000, 384),
                                   (1100, 7700, 640), (2048, 4096, 1280), (1100, 7700, 1408),
                                   (1792, 4600, 640), (1792, 4700, 640), (300, 1000, 384)])
def test_gemm_asym_x32_group_counts_exact(M, N, K):
    """The asymmetric kernel (32x32 MFMA blocks, groups processed in pairs of
    a four-group loop) over 1, 2, 3, 5, 10 and 11 groups, with M and N not
    multiples of the tile: unit scales give the oracle's integers exactly.
    1792 x 4600 has 252 tiles of 256 rows and runs the 4-wave 128-row
    instance, 1792 x 4700 (259 tiles) the 8-wave one; 300 x 1000 the 4-wave
    one with a partial last tile."""
    u, zp, qw = _asym_case(M, N, K, M + N + K)
    G = K // 128
    y = host(R.w4a4_gemm(dev(O.pack_nibbles(u)), dev(np.ones((M, G), np.float32)), dev(zp.astype(np.uint8)),
                         dev(O.pack_nibbles(qw)), dev(np.ones(N, np.float32)), act_mode="asym"))
    lv = u.reshape(M, G, 128) - zp[:, :, None]
    want = O.int_gemm(lv.reshape(M, K), qw)
    assert np.array_equal(y, want.astype(np.float32))


@pytest.mark.parametrize("M,N,K", [(1100, 7700, 1408), (2000, 4000, 384)])
def test_gemm_asym_x32_random_scales(M, N, K):
    """Random per-group scales through the same kernel: within 1e-6 of the
    oracle's float64 sum of group products."""
    u, zp, qw = _asym_case(M, N, K, 5 * M + K)
    rng = np.random.default_rng(M + K)
    sx = (rng.random((M, K // 128)) + 0.05).astype(np.float32)
    sw = (rng.random(N) * 0.01 + 1e-4).astype(np.float32)
    y = host(R.w4a4_gemm(dev(O.pack_nibbles(u)), dev(sx), dev(zp.astype(np.uint8)), dev(O.pack_nibbles(qw)),
                         dev(sw), act_mode="asym"))
    assert rel_fro(y, O.gemm_asym_f64(u, zp, sx, qw, sw)) < 1e-6


# ---------------------------------------------------------------- canaries after every output
CANARY = 0xA5
TAIL = 256


def _canaried(nbytes):
    """A device byte buffer with TAIL canary bytes after the first nbytes (16-byte aligned)."""
    t = torch.full((nbytes + TAIL,), CANARY, dtype=torch.uint8, device="cuda")
    return t


def _tail_ok(t, nbytes):
    return bool(torch.all(t[nbytes:] == CANARY).item())


def _stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("mode,block", [("sym", 128), ("sym", "full"), ("asym", 128)])
def test_rotate_quant_act_writes_nothing_past_its_outputs(mode, block):
    M, K = 37, 512
    x = WL.small_random(3, M, K, outlier_cols=[5], mult=30.0)
    xd = dev(x)
    G = K // 128
    nc, ns, nz = M * K // 2, 4 * (M if mode == "sym" else M * G), (M * G if mode == "asym" else 0)
    c, s = _canaried(nc), _canaried(ns)
    z = _canaried(nz) if mode == "asym" else None
    hb = 128 if block == 128 else 0
    st = _lib.call("rotate_quant_act", xd.data_ptr(), M, K, K, hb, None, 0 if mode == "sym" else 1,
                   c.data_ptr(), s.data_ptr(), None if z is None else z.data_ptr(), _stream())
    assert st == 0, _lib.last_error()
    assert _tail_ok(c, nc) and _tail_ok(s, ns) and (z is None or _tail_ok(z, nz))
    codes = host(c[:nc]).reshape(M, K // 2)
    b = 128 if block == 128 else K
    if mode == "sym":
        check_sym(codes, host(s[:ns]).view(np.float32), O.quant_sym_rows(O.rotate(x, b), b))
    else:
        check_asym(codes, host(s[:ns]).view(np.float32).reshape(M, G), host(z[:nz]).reshape(M, G),
                   O.quant_asym_groups(O.rotate(x, 128), 128))


def test_quant_weight_offline_writes_nothing_past_its_outputs():
    N, K = 45, 640
    w = WL.small_random(4, N, K, std=0.02)
    wd = dev(w)
    nc, ns, ng = N * K // 2, 4 * N, 4 * N * (K // 128)
    c, s, g = _canaried(nc), _canaried(ns), _canaried(ng)
    st = _lib.call("quant_weight_offline", wd.data_ptr(), N, K, K, 128, None, c.data_ptr(), s.data_ptr(),
                   g.data_ptr(), _stream())
    assert st == 0, _lib.last_error()
    assert _tail_ok(c, nc) and _tail_ok(s, ns) and _tail_ok(g, ng)
    codes = host(c[:nc]).reshape(N, K // 2)
    ref = O.quant_weight_offline(w, 128)
    check_sym(codes, host(s[:ns]).view(np.float32), ref)
    check_gsum(host(g[:ng]).view(np.int32).reshape(N, -1), codes, ref)


def test_rotate_quant_mxfp4_writes_nothing_past_its_outputs():
    M, K = 29, 384
    x = WL.small_random(5, M, K, outlier_cols=[7], mult=30.0)
    xd = dev(x)
    nc, ne = M * K // 2, M * K // 32
    c, e = _canaried(nc), _canaried(ne)
    st = _lib.call("rotate_quant_mxfp4", xd.data_ptr(), M, K, K, 128, None, c.data_ptr(), e.data_ptr(),
                   _stream())
    assert st == 0, _lib.last_error()
    assert _tail_ok(c, nc) and _tail_ok(e, ne)
    check_mx(host(c[:nc]).reshape(M, -1), host(e[:ne]).reshape(M, -1), O.rotate_mx_quant(x, 128))


def test_kv_rotate_quant4_writes_nothing_past_its_outputs():
    B, H, S, D = 2, 3, 21, 128
    kv = WL.kv(B=B, H=H, S=S)["KV"]
    kd = dev(kv)
    n = B * H * S
    c, s, z = _canaried(n * 64), _canaried(4 * n), _canaried(n)
    st = _lib.call("kv_rotate_quant4", kd.data_ptr(), B, H, S, D, H * S * D, S * D, D, None, c.data_ptr(),
                   s.data_ptr(), z.data_ptr(), _stream())
    assert st == 0, _lib.last_error()
    assert _tail_ok(c, n * 64) and _tail_ok(s, 4 * n) and _tail_ok(z, n)
    ref = O.kv_rotate_quant(kv)
    flat = dict(ref, scale=ref["scale"].reshape(-1, 1), zp=ref["zp"].reshape(-1, 1))
    check_asym(host(c[:n * 64]).reshape(-1, 64), host(s[:4 * n]).view(np.float32).reshape(-1, 1),
               host(z[:n]).reshape(-1, 1), flat)


@pytest.mark.parametrize("M,N,K,mode", [(3, 40, 256, "sym"), (37, 130, 384, "sym"), (300, 136, 256, "sym"),
                                        (37, 130, 384, "asym")])
def test_gemm_writes_no_row_past_M(M, N, K, mode):
    """Rows M and M+1 of a taller output buffer stay untouched (decode,
    64-row and asymmetric kernels)."""
    G = K // 128
    u, zp, qw = _asym_case(M, N, K, M + N)
    qa = _codes(M, M, K)
    y = torch.full((M + 2, N), -3.0, dtype=torch.float32, device="cuda")
    if mode == "sym":
        R.w4a4_gemm(dev(O.pack_nibbles(qa)), dev(np.ones(M, np.float32)), None, dev(O.pack_nibbles(qw)),
                    dev(np.ones(N, np.float32)), out=y[:M])
        want = O.int_gemm(qa, qw)
    else:
        R.w4a4_gemm(dev(O.pack_nibbles(u)), dev(np.ones((M, G), np.float32)), dev(zp.astype(np.uint8)),
                    dev(O.pack_nibbles(qw)), dev(np.ones(N, np.float32)), act_mode="asym", out=y[:M])
        want = O.int_gemm((u.reshape(M, G, 128) - zp[:, :, None]).reshape(M, K), qw)
    yh = host(y)
    assert np.all(yh[M:] == -3.0)
    assert np.array_equal(yh[:M], want.astype(np.float32))
