"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

from rotation_w4a4_quantization_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a4.h")


def _declared():
    src = open(HEADER).read()
    return re.findall(r"W4A4_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("rotate_quant_act", "quant_weight_offline", "w4a4_gemm", "kv_rotate_quant4",
              "w4a4_last_error", "w4a4_abi_version", "w4a4_time_next_launch", "kv4_attention_decode",
              "rotate_quant_mxfp4", "mxfp4_gemm", "w4a4_decode_fused", "kv4_attention_decode_ws",
              "kv4_attention_workspace_bytes", "kv4_attention_decode_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for n in _declared():
        assert hasattr(lib, n), n
    assert lib.w4a4_abi_version() == 6
    src = open(HEADER).read()
    assert int(re.search(r"#define W4A4_ABI_VERSION (\d+)", src).group(1)) == lib.w4a4_abi_version()


def test_no_internal_symbols_exported():
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read().split("\n")
    names = {ln.split()[-1] for ln in out if ln.strip() and ln.split()[1] in ("T", "W")}
    names = {n for n in names if not n.startswith("_")}
    assert names == set(_declared())


class _Buf:
    """16-byte aligned host scratch used only as a non-NULL pointer value
    (validation fails before anything is read)."""

    def __init__(self, n=1 << 16):
        self.raw = ctypes.create_string_buffer(n + 32)
        self.a = (ctypes.addressof(self.raw) + 15) // 16 * 16


B = _Buf()
A = B.a
NUL = None


@pytest.mark.parametrize("args,status", [
    ((NUL, 4, 128, 128, 128, NUL, 0, A, A, NUL, NUL), _lib.W4A4_ERR_NULL),
    ((A, 4, 128, 128, 128, NUL, 0, NUL, A, NUL, NUL), _lib.W4A4_ERR_NULL),
    ((A, 4, 128, 128, 128, NUL, 0, A, NUL, NUL, NUL), _lib.W4A4_ERR_NULL),
    ((A, 4, 100, 128, 128, NUL, 0, A, A, NUL, NUL), _lib.W4A4_ERR_SHAPE),       # K % 128
    ((A, 4, 0, 128, 128, NUL, 0, A, A, NUL, NUL), _lib.W4A4_ERR_SHAPE),
    ((A, 4, 32768, 32768, 128, NUL, 0, A, A, NUL, NUL), _lib.W4A4_ERR_SHAPE),  # K > 16384
    ((A, -1, 128, 128, 128, NUL, 0, A, A, NUL, NUL), _lib.W4A4_ERR_SHAPE),
    ((A, 4, 256, 128, 128, NUL, 0, A, A, NUL, NUL), _lib.W4A4_ERR_SHAPE),       # ldx < K
    ((A, 4, 384, 384, 0, NUL, 0, A, A, NUL, NUL), _lib.W4A4_ERR_SHAPE),         # full needs 2^p
    ((A, 4, 128, 132, 128, NUL, 0, A, A, NUL, NUL), _lib.W4A4_ERR_ALIGN),       # ldx % 8
    ((A + 2, 4, 128, 128, 128, NUL, 0, A, A, NUL, NUL), _lib.W4A4_ERR_ALIGN),
    ((A, 4, 128, 128, 64, NUL, 0, A, A, NUL, NUL), _lib.W4A4_ERR_MODE),         # had_block
    ((A, 4, 128, 128, 128, NUL, 2, A, A, NUL, NUL), _lib.W4A4_ERR_MODE),        # act_mode
    ((A, 4, 128, 128, 128, NUL, 0, A, A, A, NUL), _lib.W4A4_ERR_MODE),          # zeros in sym
    ((A, 4, 128, 128, 128, NUL, 1, A, A, NUL, NUL), _lib.W4A4_ERR_MODE),        # no zeros in asym
    ((A, 4, 256, 256, 0, NUL, 1, A, A, A, NUL), _lib.W4A4_ERR_MODE),            # asym + full
    ((A, 0, 128, 128, 128, NUL, 0, A, A, NUL, NUL), _lib.W4A4_OK),              # M == 0: no-op
    ((NUL, 0, 128, 128, 128, NUL, 0, NUL, NUL, NUL, NUL), _lib.W4A4_OK),        # M == 0, NULL buffers
    ((NUL, 0, 100, 128, 128, NUL, 0, NUL, NUL, NUL, NUL), _lib.W4A4_ERR_SHAPE),  # sizes still checked
    ((A, 4, 128, 128, 128, A + 2, 0, A, A, NUL, NUL), _lib.W4A4_ERR_ALIGN),  # signs alignment
])
def test_rotate_quant_act_validation(args, status):
    assert _lib.call("rotate_quant_act", *args) == status
    assert (_lib.last_error() == "") == (status == _lib.W4A4_OK)


@pytest.mark.parametrize("args,status", [
    ((NUL, 4, 128, 128, 128, NUL, A, A, NUL, NUL), _lib.W4A4_ERR_NULL),
    ((A, 4, 128, 128, 128, NUL, A, NUL, NUL, NUL), _lib.W4A4_ERR_NULL),
    ((A, 4, 200, 200, 128, NUL, A, A, NUL, NUL), _lib.W4A4_ERR_SHAPE),
    ((A, 4, 128, 128, 7, NUL, A, A, NUL, NUL), _lib.W4A4_ERR_MODE),
    ((A, 4, 128, 128, 128, NUL, A, A, A + 4, NUL), _lib.W4A4_ERR_ALIGN),
    ((A, 0, 128, 128, 128, NUL, A, A, A, NUL), _lib.W4A4_OK),
    ((A, 4, 128, 128, 128, A + 8, A, A, NUL, NUL), _lib.W4A4_ERR_ALIGN),      # signs alignment
])
def test_quant_weight_offline_validation(args, status):
    assert _lib.call("quant_weight_offline", *args) == status


@pytest.mark.parametrize("args,status", [
    ((NUL, A, NUL, 0, A, A, NUL, 4, 4, 128, A, 4, NUL), _lib.W4A4_ERR_NULL),
    ((A, A, NUL, 0, A, A, NUL, 4, 4, 128, NUL, 4, NUL), _lib.W4A4_ERR_NULL),
    ((A, A, NUL, 1, A, A, NUL, 4, 4, 128, A, 4, NUL), _lib.W4A4_ERR_MODE),   # asym without zeros
    ((A, A, NUL, 3, A, A, NUL, 4, 4, 128, A, 4, NUL), _lib.W4A4_ERR_MODE),
    ((A, A, NUL, 0, A, A, NUL, 4, 0, 128, A, 4, NUL), _lib.W4A4_ERR_SHAPE),  # N == 0
    ((A, A, NUL, 0, A, A, NUL, 4, 4, 96, A, 4, NUL), _lib.W4A4_ERR_SHAPE),
    ((A, A, NUL, 0, A, A, NUL, 4, 4, 128, A, 3, NUL), _lib.W4A4_ERR_SHAPE),  # ldy < N
    ((A, A, NUL, 0, A, A, NUL, 4, 4, 262144, A, 4, NUL), _lib.W4A4_ERR_SHAPE),
    ((A, A, NUL, 0, A + 8, A, NUL, 4, 4, 128, A, 4, NUL), _lib.W4A4_ERR_ALIGN),
    ((A, A, NUL, 0, A, A, NUL, 0, 4, 128, A, 4, NUL), _lib.W4A4_OK),        # M == 0: no-op
    ((NUL, NUL, NUL, 0, NUL, NUL, NUL, 0, 4, 128, NUL, 4, NUL), _lib.W4A4_OK),
])
def test_gemm_validation(args, status):
    assert _lib.call("w4a4_gemm", *args) == status


@pytest.mark.parametrize("args,status", [
    ((NUL, 1, 1, 1, 128, 128, 128, 128, NUL, A, A, A, NUL), _lib.W4A4_ERR_NULL),
    ((A, 1, 1, 1, 128, 128, 128, 128, NUL, A, A, NUL, NUL), _lib.W4A4_ERR_NULL),
    ((A, 1, 1, 1, 64, 64, 64, 64, NUL, A, A, A, NUL), _lib.W4A4_ERR_SHAPE),      # D != 128
    ((A, -1, 1, 1, 128, 128, 128, 128, NUL, A, A, A, NUL), _lib.W4A4_ERR_SHAPE),
    ((A, 1, 1, 1, 128, 128, 128, 124, NUL, A, A, A, NUL), _lib.W4A4_ERR_ALIGN),
    ((A, 1 << 16, 1 << 10, 1 << 6, 128, 128, 128, 128, NUL, A, A, A, NUL), _lib.W4A4_ERR_SHAPE),
    ((A, 0, 4, 4, 128, 128, 128, 128, NUL, A, A, A, NUL), _lib.W4A4_OK),
    ((A, 1, 1, 1, 128, 128, 128, 128, A + 4, A, A, A, NUL), _lib.W4A4_ERR_ALIGN),  # signs alignment
])
def test_kv_validation(args, status):
    assert _lib.call("kv_rotate_quant4", *args) == status


@pytest.mark.parametrize("args,status", [
    # q, kc, ks, kz, vc, vs, vz, B, H, S, D, scale, signs, out, stream
    ((NUL, A, A, A, A, A, A, 1, 2, 16, 128, 0.1, NUL, A, NUL), _lib.W4A4_ERR_NULL),
    ((A, A, A, A, A, A, NUL, 1, 2, 16, 128, 0.1, NUL, A, NUL), _lib.W4A4_ERR_NULL),
    ((A, A, A, A, A, A, A, 1, 2, 16, 128, 0.1, NUL, NUL, NUL), _lib.W4A4_ERR_NULL),
    ((A, A, A, A, A, A, A, 1, 2, 16, 64, 0.1, NUL, A, NUL), _lib.W4A4_ERR_SHAPE),     # D != 128
    ((A, A, A, A, A, A, A, 1, 2, 0, 128, 0.1, NUL, A, NUL), _lib.W4A4_ERR_SHAPE),     # S == 0
    ((A, A, A, A, A, A, A, 1, 2, 1 << 25, 128, 0.1, NUL, A, NUL), _lib.W4A4_ERR_SHAPE),
    ((A, A, A, A, A, A, A, -1, 2, 16, 128, 0.1, NUL, A, NUL), _lib.W4A4_ERR_SHAPE),
    ((A, A, A, A, A, A, A, 1, 2, 16, 128, 0.0, NUL, A, NUL), _lib.W4A4_ERR_SHAPE),    # scale <= 0
    ((A, A, A, A, A, A, A, 1, 2, 16, 128, float("nan"), NUL, A, NUL), _lib.W4A4_ERR_SHAPE),
    ((A + 4, A, A, A, A, A, A, 1, 2, 16, 128, 0.1, NUL, A, NUL), _lib.W4A4_ERR_ALIGN),
    ((A, A, A, A, A, A, A, 1, 2, 16, 128, 0.1, A + 2, A, NUL), _lib.W4A4_ERR_ALIGN),  # signs
    ((A, A, A, A, A, A, A, 0, 2, 16, 128, 0.1, NUL, A, NUL), _lib.W4A4_OK),           # B*H == 0
    ((NUL, NUL, NUL, NUL, NUL, NUL, NUL, 3, 0, 16, 128, 0.1, NUL, NUL, NUL), _lib.W4A4_OK),
])
def test_kv4_attention_validation(args, status):
    assert _lib.call("kv4_attention_decode", *args) == status


@pytest.mark.parametrize("args,status", [
    # x, M, K, ldx, had_block, signs, codes, scales, stream
    ((NUL, 4, 128, 128, 128, NUL, A, A, NUL), _lib.W4A4_ERR_NULL),
    ((A, 4, 128, 128, 128, NUL, NUL, A, NUL), _lib.W4A4_ERR_NULL),
    ((A, 4, 128, 128, 128, NUL, A, NUL, NUL), _lib.W4A4_ERR_NULL),
    ((A, 4, 160, 160, 128, NUL, A, A, NUL), _lib.W4A4_ERR_SHAPE),          # K % 128
    ((A, 4, 384, 384, 0, NUL, A, A, NUL), _lib.W4A4_ERR_SHAPE),            # full needs 2^p
    ((A, 4, 256, 128, 128, NUL, A, A, NUL), _lib.W4A4_ERR_SHAPE),          # ldx < K
    ((A, -1, 128, 128, 128, NUL, A, A, NUL), _lib.W4A4_ERR_SHAPE),
    ((A, 4, 128, 128, 32, NUL, A, A, NUL), _lib.W4A4_ERR_MODE),            # had_block
    ((A, 4, 128, 128, 128, NUL, A, A + 4, NUL), _lib.W4A4_ERR_ALIGN),
    ((A, 4, 128, 128, 128, A + 2, A, A, NUL), _lib.W4A4_ERR_ALIGN),        # signs alignment
    ((A, 4, 128, 132, 128, NUL, A, A, NUL), _lib.W4A4_ERR_ALIGN),          # ldx % 8
    ((NUL, 0, 128, 128, 128, NUL, NUL, NUL, NUL), _lib.W4A4_OK),           # M == 0: no-op
])
def test_rotate_quant_mxfp4_validation(args, status):
    assert _lib.call("rotate_quant_mxfp4", *args) == status
    assert (_lib.last_error() == "") == (status == _lib.W4A4_OK)


@pytest.mark.parametrize("args,status", [
    # xc, xe, wc, we, M, N, K, y, ldy, stream
    ((NUL, A, A, A, 4, 4, 128, A, 4, NUL), _lib.W4A4_ERR_NULL),
    ((A, NUL, A, A, 4, 4, 128, A, 4, NUL), _lib.W4A4_ERR_NULL),
    ((A, A, A, NUL, 4, 4, 128, A, 4, NUL), _lib.W4A4_ERR_NULL),
    ((A, A, A, A, 4, 4, 128, NUL, 4, NUL), _lib.W4A4_ERR_NULL),
    ((A, A, A, A, 4, 0, 128, A, 4, NUL), _lib.W4A4_ERR_SHAPE),            # N == 0
    ((A, A, A, A, 4, 4, 96, A, 4, NUL), _lib.W4A4_ERR_SHAPE),             # K % 128
    ((A, A, A, A, 4, 4, 262144, A, 4, NUL), _lib.W4A4_ERR_SHAPE),         # K too large
    ((A, A, A, A, 4, 4, 128, A, 3, NUL), _lib.W4A4_ERR_SHAPE),            # ldy < N
    ((A, A, A, A, -2, 4, 128, A, 4, NUL), _lib.W4A4_ERR_SHAPE),
    ((A, A + 4, A, A, 4, 4, 128, A, 4, NUL), _lib.W4A4_ERR_ALIGN),
    ((A, A, A, A, 4, 4, 128, A + 8, 4, NUL), _lib.W4A4_ERR_ALIGN),
    ((NUL, NUL, NUL, NUL, 0, 4, 128, NUL, 4, NUL), _lib.W4A4_OK),         # M == 0: no-op
])
def test_mxfp4_gemm_validation(args, status):
    assert _lib.call("mxfp4_gemm", *args) == status
    assert (_lib.last_error() == "") == (status == _lib.W4A4_OK)


@pytest.mark.parametrize("args,status", [
    # x, M, K, ldx, signs, w_codes, w_scales, N, y, ldy, stream
    ((NUL, 4, 256, 256, NUL, A, A, 64, A, 64, NUL), _lib.W4A4_ERR_NULL),
    ((A, 4, 256, 256, NUL, NUL, A, 64, A, 64, NUL), _lib.W4A4_ERR_NULL),
    ((A, 4, 256, 256, NUL, A, A, 64, NUL, 64, NUL), _lib.W4A4_ERR_NULL),
    ((A, 0, 256, 256, NUL, A, A, 64, A, 64, NUL), _lib.W4A4_ERR_SHAPE),      # M == 0
    ((A, 17, 256, 256, NUL, A, A, 64, A, 64, NUL), _lib.W4A4_ERR_SHAPE),     # M > 16
    ((A, 4, 200, 200, NUL, A, A, 64, A, 64, NUL), _lib.W4A4_ERR_SHAPE),      # K % 128
    ((A, 2, 16384, 16384, NUL, A, A, 64, A, 64, NUL), _lib.W4A4_ERR_SHAPE),  # K > 8192
    ((A, 16, 8192, 8192, NUL, A, A, 64, A, 64, NUL), _lib.W4A4_ERR_SHAPE),   # M * K > 65536
    ((A, 4, 256, 128, NUL, A, A, 64, A, 64, NUL), _lib.W4A4_ERR_SHAPE),      # ldx < K
    ((A, 4, 256, 260, NUL, A, A, 64, A, 64, NUL), _lib.W4A4_ERR_ALIGN),      # ldx % 8
    ((A, 4, 256, 256, NUL, A, A, 0, A, 64, NUL), _lib.W4A4_ERR_SHAPE),       # N == 0
    ((A, 4, 256, 256, NUL, A, A, 64, A, 63, NUL), _lib.W4A4_ERR_SHAPE),      # ldy < N
    ((A + 2, 4, 256, 256, NUL, A, A, 64, A, 64, NUL), _lib.W4A4_ERR_ALIGN),
    ((A, 4, 256, 256, A + 4, A, A, 64, A, 64, NUL), _lib.W4A4_ERR_ALIGN),    # signs alignment
])
def test_decode_fused_validation(args, status):
    assert _lib.call("w4a4_decode_fused", *args) == status
    assert (_lib.last_error() == "") == (status == _lib.W4A4_OK)


def test_time_next_launch_arming():
    """The timing hook needs no device: both NULL or both set; an entry point
    that fails validation disarms it (the next launch is not timed by stale events)."""
    assert _lib.call("w4a4_time_next_launch", A, NUL) == _lib.W4A4_ERR_NULL
    assert _lib.call("w4a4_time_next_launch", NUL, A) == _lib.W4A4_ERR_NULL
    assert _lib.call("w4a4_time_next_launch", NUL, NUL) == _lib.W4A4_OK
    assert _lib.call("w4a4_time_next_launch", A, A + 16) == _lib.W4A4_OK
    # a failing call consumes the armed pair; nothing reads the (host) pointers
    assert _lib.call("rotate_quant_act", A, 4, 100, 128, 128, NUL, 0, A, A, NUL, NUL) == _lib.W4A4_ERR_SHAPE
    assert _lib.call("w4a4_time_next_launch", NUL, NUL) == _lib.W4A4_OK


def test_no_device_is_a_device_error():
    """Valid arguments on a machine without a gfx950 GPU: W4A4_ERR_DEVICE, nothing launched."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = _lib.call("rotate_quant_act", A, 4, 128, 128, 128, NUL, 0, A, A, NUL, NUL)
    assert st == _lib.W4A4_ERR_DEVICE
    assert "device" in _lib.last_error()


@pytest.mark.parametrize("B,H,S,want", [
    (8, 32, 4096, 0),                      # 256 heads: single pass
    (1, 32, 4096, 32 * 8 * 528),           # ceil(256/32) = 8 ranges
    (1, 8, 32768, 8 * 32 * 528),           # 32 ranges
    (1, 1, 1 << 20, 64 * 528),             # capped at 64 ranges
    (1, 2, 700, 0),                        # S / 512 = 1: single pass
    (1, 2, 1024, 2 * 2 * 528),
    (0, 5, 100, 0),
])
def test_attention_workspace_bytes(B, H, S, want):
    assert _lib.load().kv4_attention_workspace_bytes(B, H, S) == want


@pytest.mark.parametrize("B,H,S", [(-1, 2, 10), (1, 2, 0), (1, 2, 1 << 25), (1 << 40, 1 << 30, 10)])
def test_attention_workspace_bytes_rejects(B, H, S):
    assert _lib.load().kv4_attention_workspace_bytes(B, H, S) == -1
    assert _lib.last_error()


def _ws_args(B=1, H=8, S=32768, q=A, ws=A, nbytes=1 << 30):
    return (q, A, A, A, A, A, A, B, H, S, 128, 0.088, NUL, A, ws, nbytes, NUL)


@pytest.mark.parametrize("args,status", [
    (_ws_args(nbytes=8 * 32 * 528 - 1), _lib.W4A4_ERR_SHAPE),      # workspace one byte short
    (_ws_args(ws=NUL), _lib.W4A4_ERR_NULL),
    (_ws_args(ws=A + 8), _lib.W4A4_ERR_ALIGN),
    (_ws_args(q=NUL), _lib.W4A4_ERR_NULL),
    (_ws_args(S=0), _lib.W4A4_ERR_SHAPE),
    (_ws_args(B=0, ws=NUL, nbytes=0), _lib.W4A4_OK),                 # no heads: no-op
    (_ws_args(B=8, H=32, S=4096, ws=NUL, nbytes=0), _lib.W4A4_ERR_DEVICE),   # single pass: no workspace needed
])
def test_kv4_attention_ws_validation(args, status):
    assert _lib.call("kv4_attention_decode_ws", *args) == status


@pytest.mark.parametrize("args,status", [
    ((A, A, A, A, A, A, A, 1, 8, 32768, 128, 0.088, NUL, A, NUL), _lib.W4A4_ERR_DEVICE),   # valid: reaches the device check
    ((NUL, A, A, A, A, A, A, 1, 8, 32768, 128, 0.088, NUL, A, NUL), _lib.W4A4_ERR_NULL),
    ((A, A, A, A, A, A, A, 1, 8, 0, 128, 0.088, NUL, A, NUL), _lib.W4A4_ERR_SHAPE),
    ((A, A, A, A, A, A, A, 0, 8, 100, 128, 0.088, NUL, A, NUL), _lib.W4A4_OK),             # no heads: no-op
])
def test_kv4_attention_noalloc_validation(args, status):
    assert _lib.call("kv4_attention_decode_noalloc", *args) == status
