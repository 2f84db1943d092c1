"""Two HIP streams using the library at the same time: every entry point is
stateless apart from the allocation-free attention's static scratch (whose
calls must not overlap on one GPU), and orders its work on the caller's
stream only.  The same sequences run interleaved on two streams (default
priority) must give exactly the results of running them one after another on
one stream."""
import numpy as np
import pytest

import workloads as WL

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import rotation_w4a4_quantization_amd as R

ROUNDS = 4


def _h(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _prefill(x, w):
    wc, ws, gs = R.quant_weight_offline(w, 128)
    xc, xs, _ = R.rotate_quant_act(x, 128)
    y = R.w4a4_gemm(xc, xs, None, wc, ws)
    ac, as_, az = R.rotate_quant_act(x, 128, act_mode="asym")
    ya = R.w4a4_gemm(ac, as_, az, wc, ws, gs, act_mode="asym")
    return [wc, ws, gs, xc, xs, y, ac, as_, az, ya]


def _decode(kv, q, xd, wc, ws):
    kc, ks, kz = R.kv_rotate_quant4(kv[0])
    vc, vs, vz = R.kv_rotate_quant4(kv[1])
    o1 = R.kv4_attention_decode(q, kc, ks, kz, vc, vs, vz)
    o2 = R.kv4_attention_decode_split(q, kc, ks, kz, vc, vs, vz)
    yd = R.w4a4_decode_fused(xd, wc, ws)
    return [kc, ks, kz, o1, o2, yd]


def test_two_streams_equal_serial():
    M, K, N = 1024, 2048, 1536
    B, H, S = 1, 4, 3000
    inputs = []
    for s in range(2):
        x = _h(WL.small_random(600 + s, M, K, outlier_cols=[5, 700], mult=30.0))
        w = _h(WL.small_random(610 + s, N, K, std=0.02))
        kv = _h(WL.small_random(620 + s, 2 * B * H * S, 128, outlier_cols=[3], mult=20.0).reshape(2, B, H, S, 128))
        q = _h(WL.small_random(630 + s, B * H, 128).reshape(B, H, 128))
        xd = _h(WL.small_random(640 + s, 9, K))
        inputs.append((x, w, kv, q, xd))

    def job(i):
        x, w, kv, q, xd = inputs[i]
        pre = _prefill(x, w)
        return pre + _decode(kv, q, xd, pre[0], pre[1])

    serial = [job(0), job(1)]
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    results = [[], []]
    for _ in range(ROUNDS):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                results[i].append(job(i))
    torch.cuda.synchronize()
    for i in range(2):
        for rnd, outs in enumerate(results[i]):
            for k, (a, b) in enumerate(zip(outs, serial[i])):
                assert torch.equal(a, b), f"stream {i}, round {rnd}, output {k} differs from the serial run"
