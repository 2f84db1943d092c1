"""GPU parity of w4a4_decode_fused (rotate + quantize the M <= 16 activation
rows inside the decode GEMM) through the C ABI.

The fused kernel runs the rotate kernel's own register code and scale
formulas, so its output must equal rotate_quant_act(sym, 128) followed by
w4a4_gemm bit for bit; against the oracle's end-to-end W4A4 linear it is
held to the usual 1e-3 relative Frobenius error.
"""
import numpy as np
import pytest

import oracle as O
import workloads as WL
from parity import Y_RTOL_FRO, rel_fro

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import rotation_w4a4_quantization_amd as R   # raises if libw4a4.so is missing


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def two_calls(x, wc, ws, signs=None):
    xc, xs, _ = R.rotate_quant_act(x, 128, "sym", signs=signs)
    return R.w4a4_gemm(xc, xs, None, wc, ws)


@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (4, 640, 130), (7, 4096, 257), (16, 4096, 64),
                                   (16, 2048, 4096), (8, 8192, 100), (3, 1152, 33), (16, 128, 1)])
@pytest.mark.parametrize("signed", [False, True])
def test_decode_fused_equals_two_calls(M, K, N, signed):
    s = M * 31 + K + N
    x_np = WL.small_random(s, M, K, outlier_cols=[K // 5, K - 2], mult=30.0)
    w_np = WL.small_random(s + 1, N, K, std=0.02)
    d_np = WL.hadamard_signs(K, seed=s) if signed else None
    x, w = dev(x_np), dev(w_np)
    d = dev(d_np) if signed else None
    wc, ws, _ = R.quant_weight_offline(w, 128, signs=d)
    y = R.w4a4_decode_fused(x, wc, ws, signs=d)
    y2 = two_calls(x, wc, ws, d)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), f"max diff {float((y - y2).abs().max())}"
    ref = O.w4a4_linear(x_np, w_np, 128, signs=d_np)["y"]
    assert rel_fro(y.cpu().numpy(), ref) <= Y_RTOL_FRO


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_fused_decode_config(M):
    """The decode workload: M rows like q_proj's activations against the
    4096 x 4096 q_proj weight, in the launch configuration bench times."""
    d = WL.decode(M)
    x, w = dev(d["X"]), dev(d["W"])
    wc, ws, _ = R.quant_weight_offline(w, 128)
    y = R.w4a4_decode_fused(x, wc, ws)
    y2 = two_calls(x, wc, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    ref = O.w4a4_linear(d["X"], d["W"], 128)["y"]
    r = rel_fro(y.cpu().numpy(), ref)
    print("decode M", M, "rel_fro vs oracle", r)
    assert r <= Y_RTOL_FRO


def test_decode_fused_strides_and_edges():
    """Row strides on both sides, a zero row and a row with one huge value."""
    M, K, N = 5, 1024, 96
    x_np = WL.small_random(77, M, K + 40)
    x_np[1] = 0.0
    x_np[3, :] = 0.0
    x_np[3, 500] = -60000.0
    w_np = WL.small_random(78, N, K, std=0.02)
    xt = dev(x_np)[:, :K]                                   # ldx = K + 40
    wc, ws, _ = R.quant_weight_offline(dev(w_np), 128)
    big = torch.full((M, N + 20), 3.0, dtype=torch.float32, device="cuda")
    R.w4a4_decode_fused(xt, wc, ws, out=big[:, :N])
    y2 = two_calls(xt, wc, ws)
    torch.cuda.synchronize()
    assert torch.equal(big[:, :N], y2)
    assert torch.all(big[:, N:] == 3.0)                     # columns past N untouched
    assert torch.all(big[1, :N] == 0.0)                     # a zero row gives a zero output row
