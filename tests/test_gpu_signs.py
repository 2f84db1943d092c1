"""GPU parity for the randomized Hadamard diag(d) H (the `signs` argument of
the three rotate calls) against the oracle, through the C ABI.

QuaRot page, field "Activation scheme" (randomized Hadamard); rotation page,
"The recipe" (random vs fixed Hadamard).  The signs come from
workloads.hadamard_signs; the same rules as tests/test_gpu_parity.py apply.
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
    import rotation_w4a4_quantization_amd as R


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("M,K", [(37, 384), (300, 4096), (1, 16384), (64, 2176)])
def test_signed_act_sym(M, K):
    x = WL.small_random(M + 3 * K, M, K, outlier_cols=[K // 5, K - 2], mult=30.0)
    d = WL.hadamard_signs(K, seed=K)
    blocks = [128] + ([K] if K & (K - 1) == 0 and K > 128 else [])
    for b in blocks:
        c, s, _ = R.rotate_quant_act(dev(x), 128 if b == 128 else "full", signs=dev(d))
        st = check_sym(host(c), host(s), O.quant_sym_rows(O.rotate(x, b, d), b))
        print(M, K, b, st)


@pytest.mark.parametrize("K,block", [(1024, 128), (4096, 4096)])
def test_signed_exact_class_bitexact(K, block):
    """Flipping signs keeps integer inputs integer: codes and scales stay bit-exact."""
    x = WL.exact_class(K + 1, 48, K, lim=2048, outlier_cols=[3, K // 2])
    d = WL.hadamard_signs(K, seed=7)
    c, s, _ = R.rotate_quant_act(dev(x), 128 if block == 128 else "full", signs=dev(d))
    z = O.rotate(x, block, d)
    check_sym(host(c), host(s), O.quant_sym_rows(z, block, "f32"), exact=True)
    check_sym(host(c), host(s), O.quant_sym_rows(z, block))


def test_all_plus_signs_equal_no_signs():
    x = WL.small_random(5, 40, 2048, outlier_cols=[9], mult=40.0)
    ones = np.ones(2048, np.float16)
    for hb in (128, "full"):
        a = R.rotate_quant_act(dev(x), hb)
        b = R.rotate_quant_act(dev(x), hb, signs=dev(ones))
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("M,K", [(33, 1024), (256, 8192)])
def test_signed_act_asym(M, K):
    x = WL.small_random(M * K, M, K, outlier_cols=[2, K - 9], mult=30.0)
    d = WL.hadamard_signs(K, seed=M)
    c, s, z = R.rotate_quant_act(dev(x), 128, "asym", signs=dev(d))
    check_asym(host(c), host(s), host(z), O.quant_asym_groups(O.rotate(x, 128, d), 128))


@pytest.mark.parametrize("block", [128, 4096])
def test_signed_weight_offline(block):
    w = WL.qproj_weight()[:512]
    d = WL.hadamard_signs(4096, seed=11)
    c, s, g = R.quant_weight_offline(dev(w), block if block == 128 else "full", signs=dev(d))
    c, s, g = host(c), host(s), host(g)
    ref = O.quant_weight_offline(w, block, signs=d)
    check_sym(c, s, ref)
    check_gsum(g, c, ref)


def test_signed_kv_dense_and_strided():
    kv = WL.kv(B=2, H=3, S=70)["KV"]
    d = WL.hadamard_signs(128, seed=2)
    c, s, z = R.kv_rotate_quant4(dev(kv), signs=dev(d))
    ref = O.kv_rotate_quant(kv, signs=d)
    flat = dict(ref, scale=ref["scale"].reshape(-1, 1), zp=ref["zp"].reshape(-1, 1))
    check_asym(host(c).reshape(-1, 64), host(s).reshape(-1, 1), host(z).reshape(-1, 1), flat)
    bshd = dev(np.ascontiguousarray(kv.transpose(0, 2, 1, 3)))
    c2, s2, z2 = R.kv_rotate_quant4(bshd.permute(0, 2, 1, 3), signs=dev(d))
    assert torch.equal(c, c2) and torch.equal(s, s2) and torch.equal(z, z2)


@pytest.mark.parametrize("block", [128, 4096])
def test_signed_linear_end_to_end(block):
    """q_proj rows with a shared random diagonal on X and W: the GPU product
    matches the oracle's W4A4 product and still approximates X W^T."""
    dd = WL.qproj(M=256)
    x, w = dd["X"], dd["W"][:1024]
    d = WL.hadamard_signs(4096, seed=5)
    hb = 128 if block == 128 else "full"
    xc, xs, _ = R.rotate_quant_act(dev(x), hb, signs=dev(d))
    wc, ws, _ = R.quant_weight_offline(dev(w), hb, signs=dev(d))
    y = host(R.w4a4_gemm(xc, xs, None, wc, ws))
    ref = O.w4a4_linear(x, w, block, "sym", signs=d)
    err = rel_fro(y, ref["y"])
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    print(block, "rel_fro vs oracle", err, "vs XW^T", rel_fro(y, exact))
    assert err <= Y_RTOL_FRO
    assert rel_fro(y, exact) < 0.4


def test_signs_wrong_length_rejected():
    x = dev(WL.small_random(1, 4, 256))
    with pytest.raises(ValueError):
        R.rotate_quant_act(x, 128, signs=dev(np.ones(128, np.float16)))
