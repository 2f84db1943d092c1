"""The GEMMs at the largest K they accept (131072), with every code at its
largest magnitude and unit scales, so the accumulators reach their bound and
the exact answer is known in closed form:

- symmetric: codes -7 (nibble 9) times -7 or +7 give +-49 K; the kernels hold
  256 * acc, |256 * 49 * 131072| = 1,644,167,168 < 2^31, and Y = +-49 K is an
  integer below 2^24, exact in fp32;
- asymmetric: level 15 (code 15, zero-point 0) times 7 gives 105 per element,
  16 * 105 * 128 per group, Y = 105 K, exact in fp32 at every partial sum;
- MXFP4: E2M1 6 times 6 with exponents 2^0 gives Y = 36 K, exact in fp32.

Each shape picks a different kernel instance: the decode kernel (M <= 16),
the 64-row tiles (fewer than 256 tiles of 256 rows) and the 256-row tiles."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import rotation_w4a4_quantization_amd as R

KMAX = 131072
SHAPES = [(5, 40), (100, 130), (2048, 4096)]        # decode, 64-row, 256-row instances


def _full(rows, cols, byte):
    return torch.full((rows, cols), byte, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("wbyte,sign", [(0x99, 1), (0x77, -1)])
def test_symmetric_gemm_at_max_k(M, N, wbyte, sign):
    xc = _full(M, KMAX // 2, 0x99)                  # every code -7
    wc = _full(N, KMAX // 2, wbyte)                 # -7 or +7
    xs = torch.ones(M, dtype=torch.float32, device="cuda")
    ws = torch.ones(N, dtype=torch.float32, device="cuda")
    y = R.w4a4_gemm(xc, xs, None, wc, ws)
    torch.cuda.synchronize()
    want = float(sign * 49 * KMAX)
    assert torch.all(y == want), (y.min().item(), y.max().item(), want)


@pytest.mark.parametrize("M,N", [(100, 130), (2048, 4096)])
def test_asymmetric_gemm_at_max_k(M, N):
    G = KMAX // 128
    xc = _full(M, KMAX // 2, 0xFF)                  # every code 15
    xz = torch.zeros((M, G), dtype=torch.uint8, device="cuda")
    xs = torch.ones((M, G), dtype=torch.float32, device="cuda")
    wc = _full(N, KMAX // 2, 0x77)                  # every code +7
    ws = torch.ones(N, dtype=torch.float32, device="cuda")
    y = R.w4a4_gemm(xc, xs, xz, wc, ws, act_mode="asym")
    torch.cuda.synchronize()
    assert torch.all(y == float(105 * KMAX)), (y.min().item(), y.max().item())


@pytest.mark.parametrize("M,N", SHAPES)
def test_mxfp4_gemm_at_max_k(M, N):
    xc = _full(M, KMAX // 2, 0x77)                  # E2M1 code 7 = 6.0
    wc = _full(N, KMAX // 2, 0x77)
    xe = _full(M, KMAX // 32, 127)                  # 2^0
    we = _full(N, KMAX // 32, 127)
    y = R.mxfp4_gemm(xc, xe, wc, we)
    torch.cuda.synchronize()
    assert torch.all(y == float(36 * KMAX)), (y.min().item(), y.max().item())
