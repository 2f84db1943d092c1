"""Argument checks of the Python binding that run before any device work
(CPU tensors suffice): a GEMM operand whose shape does not match M, N and K
must be refused, since the kernels size their reads from M, N and K."""
import pytest
import torch

import rotation_w4a4_quantization_amd as R

M, N, K = 6, 10, 256
G = K // 128


def _ops(mode="sym", **over):
    u8, f32 = torch.uint8, torch.float32
    d = dict(x_codes=torch.zeros((M, K // 2), dtype=u8),
             x_scales=torch.zeros((M,) if mode == "sym" else (M, G), dtype=f32),
             x_zeros=None if mode == "sym" else torch.zeros((M, G), dtype=u8),
             w_codes=torch.zeros((N, K // 2), dtype=u8),
             w_scales=torch.zeros((N,), dtype=f32),
             w_gsum=None)
    d.update(over)
    return d


def _call(mode="sym", **over):
    d = _ops(mode, **over)
    return R.w4a4_gemm(d["x_codes"], d["x_scales"], d["x_zeros"], d["w_codes"], d["w_scales"], d["w_gsum"],
                       act_mode=mode)


@pytest.mark.parametrize("mode,over", [
    ("sym", dict(x_scales=torch.zeros((M - 1,)))),                       # short per-token scales
    ("sym", dict(x_scales=torch.zeros((M, G)))),                         # per-group scales in sym mode
    ("sym", dict(w_scales=torch.zeros((N - 1,)))),                       # short weight scales
    ("sym", dict(w_scales=torch.zeros((N, 1)))),
    ("sym", dict(x_zeros=torch.zeros((M, G), dtype=torch.uint8))),       # zeros in sym mode
    ("asym", dict(x_scales=torch.zeros((M,)))),                          # per-token scales in asym mode
    ("asym", dict(x_zeros=torch.zeros((M, G - 1), dtype=torch.uint8))),
    ("asym", dict(x_zeros=torch.zeros((G, M), dtype=torch.uint8).t())),  # right shape, not contiguous
    ("asym", dict(x_zeros=None)),
    ("sym", dict(w_codes=torch.zeros((N, K // 2 + 64), dtype=torch.uint8))),   # K mismatch
    ("sym", dict(x_codes=torch.zeros((M, K // 2, 1), dtype=torch.uint8))),
    ("sym", dict(w_gsum=torch.zeros((N, G + 1), dtype=torch.int32))),
    ("sym", dict(x_scales=torch.zeros((2 * M,))[::2])),                 # non-contiguous scales
])
def test_gemm_refuses_mismatched_operands(mode, over):
    with pytest.raises(ValueError):
        _call(mode, **over)


@pytest.mark.parametrize("mode,over", [
    ("sym", dict(x_scales=torch.zeros((M,), dtype=torch.float16))),
    ("asym", dict(x_zeros=torch.zeros((M, G), dtype=torch.int32))),
    ("sym", dict(w_gsum=torch.zeros((N, G), dtype=torch.int64))),
])
def test_gemm_refuses_wrong_dtypes(mode, over):
    with pytest.raises(TypeError):
        _call(mode, **over)


@pytest.mark.parametrize("mode", ["sym", "asym"])
def test_gemm_well_formed_host_tensors_fail_only_on_the_device_check(mode):
    """Shapes right, tensors on the host: the binding gets past every shape
    rule and stops at the device rule (nothing is launched)."""
    with pytest.raises(TypeError, match="CUDA"):
        _call(mode, w_gsum=torch.zeros((N, G), dtype=torch.int32))
