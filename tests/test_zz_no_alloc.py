"""kv4_attention_decode_noalloc (split decode attention with the partial
states in the library's static device scratch) against
kv4_attention_decode_ws (the same kernels with a caller's workspace),
through the C ABI: two calls in a row, the second smaller, each equal to the
workspace entry point's output bit for bit and to the oracle within the
same-codes bound of the attention tests (1e-4 relative)."""
import math

import numpy as np
import pytest

import oracle as O
import workloads as WL
from parity import rel_fro

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    from rotation_w4a4_quantization_amd import _lib


def _cache(B, H, S, seed):
    k = WL.small_random(seed, B * H * S, 128, outlier_cols=[3, 90], mult=20.0).reshape(B, H, S, 128)
    v = WL.small_random(seed + 1, B * H * S, 128).reshape(B, H, S, 128)
    q = WL.small_random(seed + 2, B * H, 128).reshape(B, H, 128)
    kq, vq = O.kv_rotate_quant(k), O.kv_rotate_quant(v)
    for d in (kq, vq):
        d["scale"] = d["scale"].astype(np.float32)
    return q, kq, vq


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _call(name, B, H, S, t, out, extra=()):
    stream = torch.cuda.current_stream().cuda_stream
    st = _lib.call(name, t[0].data_ptr(), *(x.data_ptr() for x in t[1:]), B, H, S, 128,
                   1 / math.sqrt(128), None, out.data_ptr(), *extra, stream)
    assert st == 0, f"{name}: {_lib.last_error()}"


@pytest.mark.parametrize("first,second", [((1, 8, 8192), (1, 2, 3000)), ((2, 4, 4096), (1, 3, 1100))])
def test_noalloc_matches_workspace_entry_point(first, second):
    lib = _lib.load()
    for B, H, S in (first, second):
        print("noalloc case", B, H, S, flush=True)
        q, kq, vq = _cache(B, H, S, 31 * S + H)
        t = [_dev(q)] + [_dev(d[key]) for d in (kq, vq) for key in ("packed", "scale", "zp")]
        need = lib.kv4_attention_workspace_bytes(B, H, S)
        assert 0 < need <= 512 * 1024
        ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
        o_ws = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
        o_na = torch.full((B, H, 128), float("nan"), dtype=torch.float32, device="cuda")
        _call("kv4_attention_decode_ws", B, H, S, t, o_ws, (ws.data_ptr(), need))
        _call("kv4_attention_decode_noalloc", B, H, S, t, o_na)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws)
        want = O.kv4_attention_decode(q, kq["packed"], kq["scale"], kq["zp"], vq["packed"], vq["scale"],
                                      vq["zp"], 1 / math.sqrt(128))
        err = rel_fro(o_na.cpu().numpy(), want)
        print("  rel_fro vs oracle", err)
        assert err <= 1e-4


def test_noalloc_single_pass_shape():
    """Enough heads for the single pass: no scratch used, same output."""
    B, H, S = 4, 64, 600
    q, kq, vq = _cache(B, H, S, 5)
    t = [_dev(q)] + [_dev(d[key]) for d in (kq, vq) for key in ("packed", "scale", "zp")]
    assert _lib.load().kv4_attention_workspace_bytes(B, H, S) == 0
    o1 = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(o1)
    _call("kv4_attention_decode", B, H, S, t, o1)
    _call("kv4_attention_decode_noalloc", B, H, S, t, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
