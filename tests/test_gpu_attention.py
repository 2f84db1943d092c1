"""GPU parity of kv4_attention_decode (decode attention over the rotated INT4
KV cache) against the oracle, through the C ABI.

QuaRot page, field "Activation scheme" (the KV cache and parts of attention
are rotated).  With identical codes on both sides the GPU's fp32 arithmetic
is the only difference: scores are sums of 128 fp32 products, the softmax
weights carry exp2 rounding, and the output is a sum over S tokens, so the
relative error is a few 1e-6 for S <= 4096; the bound below is 1e-4.  From
fp16 inputs (each side quantizing the cache itself) codes may differ at
rounding ties, and the output bound is the 1e-3 of the other dequantized
results.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as WL
from parity import Y_RTOL_FRO, rel_fro

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

if torch.cuda.is_available():
    import rotation_w4a4_quantization_amd as R

SAME_CODES_RTOL = 1e-4


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _kvq(x, signs=None):
    """The oracle's KV quantization with its scales rounded to fp32, the dtype
    the GPU reads: both sides then attend over identical codes and scales."""
    d = O.kv_rotate_quant(x, signs=signs)
    d["scale"] = d["scale"].astype(np.float32)
    return d


def _cache(B, H, S, seed):
    k = WL.small_random(seed, B * H * S, 128, outlier_cols=[3, 90], mult=20.0).reshape(B, H, S, 128)
    v = WL.small_random(seed + 1, B * H * S, 128).reshape(B, H, S, 128)
    q = WL.small_random(seed + 2, B * H, 128).reshape(B, H, 128)
    return q, k, v


@pytest.mark.parametrize("B,H,S", [(1, 1, 1), (1, 2, 5), (2, 3, 100), (1, 4, 1000), (2, 2, 4097)])
@pytest.mark.parametrize("with_signs", [False, True])
def test_attention_same_codes(B, H, S, with_signs):
    q, k, v = _cache(B, H, S, B * 1000 + H * 10 + S)
    d = WL.hadamard_signs(128, seed=S) if with_signs else None
    kq = _kvq(k, signs=d)
    vq = _kvq(v, signs=d)
    scale = 1 / math.sqrt(128)
    o = R.kv4_attention_decode(dev(q), dev(kq["packed"]), dev(kq["scale"]), dev(kq["zp"]),
                               dev(vq["packed"]), dev(vq["scale"]), dev(vq["zp"]), scale,
                               signs=None if d is None else dev(d))
    want = O.kv4_attention_decode(q, kq["packed"], kq["scale"], kq["zp"], vq["packed"], vq["scale"],
                                  vq["zp"], scale, signs=d)
    err = rel_fro(host(o), want)
    print(B, H, S, with_signs, "rel_fro", err)
    assert err <= SAME_CODES_RTOL


def test_attention_single_token_is_the_value():
    """S = 1: the softmax weight is 1 and the output is the dequantized value rotated back."""
    q, k, v = _cache(1, 3, 1, 77)
    kq, vq = _kvq(k), _kvq(v)
    o = host(R.kv4_attention_decode(dev(q), dev(kq["packed"]), dev(kq["scale"]), dev(kq["zp"]),
                                    dev(vq["packed"]), dev(vq["scale"]), dev(vq["zp"])))
    u = O.unpack_nibbles(vq["packed"].reshape(-1, 64), signed=False)
    vhat = O.dequant_asym_groups(u, vq["scale"].reshape(-1, 1), vq["zp"].reshape(-1, 1), 128)
    want = O.rotate_normalized(vhat, 128).reshape(1, 3, 128)        # H is symmetric: Q^T = Q
    assert rel_fro(o, want) <= SAME_CODES_RTOL


def test_attention_sharp_softmax():
    """A large softmax scale: the running maximum moves a lot; still same-codes exact to 1e-4."""
    q, k, v = _cache(1, 2, 700, 5)
    kq, vq = _kvq(k), _kvq(v)
    o = R.kv4_attention_decode(dev(q), dev(kq["packed"]), dev(kq["scale"]), dev(kq["zp"]),
                               dev(vq["packed"]), dev(vq["scale"]), dev(vq["zp"]), 2.0)
    want = O.kv4_attention_decode(q, kq["packed"], kq["scale"], kq["zp"], vq["packed"], vq["scale"],
                                  vq["zp"], 2.0)
    assert rel_fro(host(o), want) <= SAME_CODES_RTOL


def test_attention_end_to_end_from_fp16():
    """GPU kv_rotate_quant4 + GPU attention vs the oracle's own quantization and attention."""
    q, k, v = _cache(2, 2, 513, 9)
    d = WL.hadamard_signs(128, seed=4)
    kc, ks, kz = R.kv_rotate_quant4(dev(k), signs=dev(d))
    vc, vs, vz = R.kv_rotate_quant4(dev(v), signs=dev(d))
    o = host(R.kv4_attention_decode(dev(q), kc, ks, kz, vc, vs, vz, signs=dev(d)))
    kq, vq = O.kv_rotate_quant(k, signs=d), O.kv_rotate_quant(v, signs=d)
    want = O.kv4_attention_decode(q, kq["packed"], kq["scale"], kq["zp"], vq["packed"], vq["scale"],
                                  vq["zp"], 1 / math.sqrt(128), signs=d)
    err = rel_fro(o, want)
    print("end to end rel_fro", err, "vs fp16 attention",
          rel_fro(o, O.attention_decode_f64(q, k, v, 1 / math.sqrt(128))))
    assert err <= Y_RTOL_FRO


def test_attention_full_config_all_heads():
    """The KV config (8 x 32 x 4096 x 128) at its full launch (256 heads): the
    oracle quantizes the cache, one batch row at a time; the GPU attends over
    those codes; all 256 (batch, head) outputs checked against the oracle."""
    kv = WL.kv()["KV"]
    vv = np.ascontiguousarray(kv[:, ::-1])               # a second cache: heads reversed
    q = WL.small_random(123, 8 * 32, 128).reshape(8, 32, 128)
    kqs = [_kvq(kv[b][None]) for b in range(8)]
    vqs = [_kvq(vv[b][None]) for b in range(8)]
    cat = lambda ds, key: np.concatenate([d[key] for d in ds], axis=0)
    args = [dev(cat(ds, key)) for ds in (kqs, vqs) for key in ("packed", "scale", "zp")]
    o = host(R.kv4_attention_decode(dev(q), *args))
    worst = 0.0
    for b in range(8):
        kq, vq = kqs[b], vqs[b]
        want = O.kv4_attention_decode(q[b][None], kq["packed"], kq["scale"], kq["zp"], vq["packed"],
                                      vq["scale"], vq["zp"], 1 / math.sqrt(128))
        for h in range(32):
            worst = max(worst, rel_fro(o[b, h], want[0, h]))
    print("all 256 heads, worst rel_fro", worst)
    assert worst <= SAME_CODES_RTOL


# ---------------------------------------------------------------- tokens split over workgroups
def _split_and_single(q, kq, vq, scale, d=None):
    a = [dev(q), dev(kq["packed"]), dev(kq["scale"]), dev(kq["zp"]), dev(vq["packed"]), dev(vq["scale"]),
         dev(vq["zp"]), scale]
    sg = None if d is None else dev(d)
    return host(R.kv4_attention_decode_split(*a, signs=sg)), host(R.kv4_attention_decode(*a, signs=sg))


@pytest.mark.parametrize("B,H,S", [(1, 2, 1024), (1, 1, 5000), (1, 8, 4097), (2, 3, 3000), (1, 4, 1000)])
@pytest.mark.parametrize("with_signs", [False, True])
def test_attention_split_same_codes(B, H, S, with_signs):
    """Few heads, tokens split into ranges (ragged last range, and one case
    below the split threshold): same-codes bound against the oracle."""
    q, k, v = _cache(B, H, S, 7 * S + H)
    d = WL.hadamard_signs(128, seed=H) if with_signs else None
    kq, vq = _kvq(k, signs=d), _kvq(v, signs=d)
    scale = 1 / math.sqrt(128)
    o, o1 = _split_and_single(q, kq, vq, scale, d)
    want = O.kv4_attention_decode(q, kq["packed"], kq["scale"], kq["zp"], vq["packed"], vq["scale"],
                                  vq["zp"], scale, signs=d)
    print(B, H, S, "ranges", R.kv4_attention_workspace_bytes(B, H, S) // (528 * B * H),
          "split", rel_fro(o, want), "single", rel_fro(o1, want))
    assert rel_fro(o, want) <= SAME_CODES_RTOL


def test_attention_split_sharp_softmax():
    """A large softmax scale: range maxima far apart, the merge rescales by 2^(m_k - M)."""
    q, k, v = _cache(1, 2, 2600, 15)
    kq, vq = _kvq(k), _kvq(v)
    o, _ = _split_and_single(q, kq, vq, 2.0)
    want = O.kv4_attention_decode(q, kq["packed"], kq["scale"], kq["zp"], vq["packed"], vq["scale"],
                                  vq["zp"], 2.0)
    assert rel_fro(o, want) <= SAME_CODES_RTOL


def test_attention_split_long_context():
    """1 x 8 heads x 32768 tokens (32 ranges per head), every head checked;
    a caller-given workspace is used as is."""
    q, k, v = _cache(1, 8, 32768, 21)
    kq, vq = _kvq(k), _kvq(v)
    need = R.kv4_attention_workspace_bytes(1, 8, 32768)
    assert need == 8 * 32 * 528
    ws = torch.full((need + 64,), 0x7F, dtype=torch.uint8, device="cuda")
    a = [dev(q), dev(kq["packed"]), dev(kq["scale"]), dev(kq["zp"]), dev(vq["packed"]), dev(vq["scale"]),
         dev(vq["zp"])]
    o = host(R.kv4_attention_decode_split(*a, workspace=ws))
    assert np.all(host(ws[need:]) == 0x7F), "workspace written past its size"
    want = O.kv4_attention_decode(q, kq["packed"], kq["scale"], kq["zp"], vq["packed"], vq["scale"],
                                  vq["zp"], 1 / math.sqrt(128))
    worst = max(rel_fro(o[0, h], want[0, h]) for h in range(8))
    print("long context, worst head rel_fro", worst)
    assert worst <= SAME_CODES_RTOL


def test_attention_split_workspace_too_small_rejected():
    q, k, v = _cache(1, 2, 1024, 3)
    kq, vq = _kvq(k), _kvq(v)
    ws = torch.empty((R.kv4_attention_workspace_bytes(1, 2, 1024) - 16,), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="workspace"):
        R.kv4_attention_decode_split(dev(q), dev(kq["packed"]), dev(kq["scale"]), dev(kq["zp"]),
                                     dev(vq["packed"]), dev(vq["scale"]), dev(vq["zp"]), workspace=ws)
