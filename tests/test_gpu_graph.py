"""The entry points under HIP graph capture: every launch the library makes is
a plain kernel on the caller's stream (no memset, copy, allocation or host
synchronization inside an entry point), so a caller can capture a layer once
and replay it.  Each captured sequence is replayed several times with new
data in its static inputs, the same calls run eagerly in between (into
their own outputs), and every replay must equal the eager result bit for
bit.

Sequences: the prefill linear layer (rotate_quant_act + w4a4_gemm, symmetric
with 128-blocks and full width, asymmetric per-group), the KV step with the
three decode-attention entry points (single pass, split with a caller
workspace, split with the library's static scratch), the fused decode
linear, and the MXFP4 pair."""
import numpy as np
import pytest

import workloads as WL

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import rotation_w4a4_quantization_amd as R

REPLAYS = 3


def _h(a):
    return torch.from_numpy(np.ascontiguousarray(a))


def _capture_and_check(static_inputs, new_inputs, fn):
    """Capture fn(*static_inputs) in a graph; for each trial copy new data into
    the static inputs, replay, run fn eagerly on the same inputs, and compare."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(*static_inputs)                      # first calls (device set-up) outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn(*static_inputs)
    torch.cuda.synchronize()
    assert len(new_inputs) >= REPLAYS
    for trial in range(REPLAYS):
        for dst, src in zip(static_inputs, new_inputs[trial]):
            if src is not None:
                dst.copy_(src.to(dst.device), non_blocking=False)
        g.replay()
        ref = fn(*static_inputs)               # eager work between the replays
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            assert o.shape == e.shape and o.dtype == e.dtype
            assert torch.equal(o, e), f"replay {trial}, output {i} differs from the eager call"
    return outs


def _mats(seed, rows, cols, n, **kw):
    return [_h(WL.small_random(seed + 7 * t, rows, cols, **kw)) for t in range(n)]


@pytest.mark.parametrize("M,K,N,had,mode", [(300, 1152, 640, 128, "sym"), (2048, 1024, 4096, 128, "sym"),
                                            (300, 1024, 640, "full", "sym"), (300, 1152, 640, 128, "asym")])
def test_prefill_linear_graph(M, K, N, had, mode):
    w = _h(WL.small_random(11, N, K, std=0.02)).cuda()
    wc, ws, gs = R.quant_weight_offline(w, had)
    xs = _mats(100, M, K, REPLAYS + 1, outlier_cols=[3, K - 5], mult=30.0)
    x = xs[0].cuda()

    def layer(x):
        c, s, z = R.rotate_quant_act(x, had, act_mode=mode)
        out = R.w4a4_gemm(c, s, z, wc, ws, gs if mode == "asym" else None, act_mode=mode)
        return c, s, out if z is None else torch.cat([out.flatten(), z.float().flatten()])

    outs = _capture_and_check([x], [[xs[t + 1]] for t in range(REPLAYS)], layer)
    first = layer(xs[1].cuda())
    torch.cuda.synchronize()
    assert not torch.equal(outs[2], first[2]), "replays did not see the new inputs"


def test_kv_and_decode_attention_graph():
    B, H, S = 2, 4, 1500                                    # few heads: the split path takes 3 ranges
    signs = _h(WL.hadamard_signs(128, seed=5)).cuda()
    kvs = [_h(WL.small_random(200 + t, 2 * B * H * S, 128, outlier_cols=[3, 90], mult=20.0)
              .reshape(2, B, H, S, 128)) for t in range(REPLAYS + 1)]
    qs = [_h(WL.small_random(300 + t, B * H, 128).reshape(B, H, 128)) for t in range(REPLAYS + 1)]
    kv, q = kvs[0].cuda(), qs[0].cuda()
    need = R.kv4_attention_workspace_bytes(B, H, S)
    assert need > 0
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")

    def step(kv, q):
        kc, ks, kz = R.kv_rotate_quant4(kv[0], signs=signs)
        vc, vs, vz = R.kv_rotate_quant4(kv[1], signs=signs)
        a = R.kv4_attention_decode(q, kc, ks, kz, vc, vs, vz, signs=signs)
        b = R.kv4_attention_decode_split(q, kc, ks, kz, vc, vs, vz, signs=signs, workspace=ws)
        c = R.kv4_attention_decode_noalloc(q, kc, ks, kz, vc, vs, vz, signs=signs)
        return kc, ks, kz, a, b, c

    _capture_and_check([kv, q], [[kvs[t + 1], qs[t + 1]] for t in range(REPLAYS)], step)


@pytest.mark.parametrize("M", [1, 7, 16])
def test_fused_decode_graph(M):
    K, N = 1024, 640
    w = _h(WL.small_random(12, N, K, std=0.02)).cuda()
    wc, ws, _ = R.quant_weight_offline(w, 128, with_gsum=False)
    xs = _mats(400, M, K, REPLAYS + 1, outlier_cols=[9], mult=30.0)
    x = xs[0].cuda()

    def dec(x):
        return (R.w4a4_decode_fused(x, wc, ws),)

    _capture_and_check([x], [[xs[t + 1]] for t in range(REPLAYS)], dec)


def test_mxfp4_graph():
    M, K, N = 300, 1152, 640
    w = _h(WL.small_random(13, N, K, std=0.02)).cuda()
    wm, we = R.rotate_quant_mxfp4(w, 128)
    xs = _mats(500, M, K, REPLAYS + 1, outlier_cols=[3], mult=30.0)
    x = xs[0].cuda()

    def mx(x):
        c, e = R.rotate_quant_mxfp4(x, 128)
        return c, e, R.mxfp4_gemm(c, e, wm, we)

    _capture_and_check([x], [[xs[t + 1]] for t in range(REPLAYS)], mx)
