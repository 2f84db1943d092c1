"""The GPU-vs-oracle comparison rules themselves (CPU): they accept the
oracle's own output and reject planted mistakes of the kinds a kernel could
make (a wrong code away from a tie, a wrong exponent, swapped nibbles)."""
import numpy as np
import pytest

import oracle as O
import workloads as WL
from parity import check_asym, check_mx, check_sym, near_mx_tie


@pytest.fixture(scope="module")
def mx_ref():
    x = WL.small_random(404, 24, 512, outlier_cols=[5, 300], mult=30.0)
    return O.rotate_mx_quant(x, 128)


def test_check_mx_accepts_the_oracle(mx_ref):
    st = check_mx(mx_ref["packed"], mx_ref["scale_byte"], mx_ref)
    assert st["flips"] == 0 and st["scale_flips"] == 0
    x = WL.exact_class(404, 24, 512, lim=2048, outlier_cols=[5, 300])
    r32 = O.rotate_mx_quant(x, 128, decide="f32")
    st = check_mx(r32["packed"], r32["scale_byte"], r32, exact=True)
    assert st["flips"] == 0 and st["scale_flips"] == 0
    with pytest.raises(AssertionError):            # an exact comparison needs the exact-fp32 mode
        check_mx(mx_ref["packed"], mx_ref["scale_byte"], mx_ref, exact=True)


def test_check_mx_rejects_a_code_away_from_a_midpoint(mx_ref):
    c = mx_ref["codes"].copy()
    t = mx_ref["y"].reshape(c.shape[0], -1, 32) / np.exp2(mx_ref["scale_e"])[..., None]
    t = t.reshape(c.shape)
    i, j = np.argwhere(((c & 7) > 0) & ((c & 7) < 7) & ~near_mx_tie(t))[0]
    c[i, j] += 1                                  # one magnitude step up, far from a tie
    with pytest.raises(AssertionError):
        check_mx(O.pack_nibbles(c), mx_ref["scale_byte"], mx_ref)


def test_check_mx_rejects_a_wrong_exponent(mx_ref):
    b = mx_ref["scale_byte"].copy()
    b[3, 2] += 1
    with pytest.raises(AssertionError):
        check_mx(mx_ref["packed"], b, mx_ref)


def test_check_mx_rejects_swapped_nibbles(mx_ref):
    p = mx_ref["packed"].copy()
    i, j = np.argwhere((p & 0xF) != (p >> 4))[0]
    p[i, j] = ((p[i, j] & 0xF) << 4) | (p[i, j] >> 4)
    with pytest.raises(AssertionError):
        check_mx(p, mx_ref["scale_byte"], mx_ref)


def test_check_mx_rejects_a_sign_flip(mx_ref):
    c = mx_ref["codes"].copy()
    i, j = np.argwhere((c & 7) >= 2)[0]
    c[i, j] ^= 8
    with pytest.raises(AssertionError):
        check_mx(O.pack_nibbles(c), mx_ref["scale_byte"], mx_ref)


def test_check_sym_accepts_the_oracle_and_rejects_a_flip():
    x = WL.small_random(405, 16, 256, outlier_cols=[3], mult=40.0)
    ref = O.quant_sym_rows(O.rotate(x, 128), 128)
    packed = O.pack_nibbles(ref["codes"])
    check_sym(packed, ref["scale"].astype(np.float32), ref)
    r32 = O.quant_sym_rows(O.rotate(x, 128), 128, "f32")
    check_sym(O.pack_nibbles(r32["codes"]), r32["scale"], r32, exact=True)
    c = ref["codes"].astype(np.int64).copy()
    far = np.abs(np.abs(ref["t"] - np.floor(ref["t"])) - 0.5) > 0.1
    i, j = np.argwhere(far & (np.abs(c) < 7))[0]
    c[i, j] += 1
    with pytest.raises(AssertionError):
        check_sym(O.pack_nibbles(c), ref["scale"], ref)


def test_check_asym_accepts_the_oracle_and_rejects_mistakes():
    x = WL.small_random(406, 12, 512, outlier_cols=[7, 300], mult=25.0)
    z = O.rotate(x, 128)
    ref = O.quant_asym_groups(z, 128)
    packed = O.pack_nibbles(ref["codes"])
    st = check_asym(packed, ref["scale"].astype(np.float32), ref["zp"], ref)
    assert st["flips"] == 0 and st["zp_flips"] == 0
    r32 = O.quant_asym_groups(z, 128, mode="f32")
    check_asym(O.pack_nibbles(r32["codes"]), r32["scale"], r32["zp"], r32, exact=True)
    # a level moved by one away from any tie
    c = ref["codes"].astype(np.int64).copy()
    far = np.abs(np.abs(ref["t"] - np.floor(ref["t"])) - 0.5) > 0.1
    i, j = np.argwhere(far & (c < 15))[0]
    c[i, j] += 1
    with pytest.raises(AssertionError):
        check_asym(O.pack_nibbles(c), ref["scale"].astype(np.float32), ref["zp"], ref)
    # a zero-point moved away from its tie (codes unchanged)
    zp = ref["zp"].copy()
    zfar = np.abs(np.abs(ref["t_zp"] - np.floor(ref["t_zp"])) - 0.5) > 0.1
    gi, gj = np.argwhere(zfar & (zp < 15))[0]
    zp[gi, gj] += 1
    with pytest.raises(AssertionError):
        check_asym(packed, ref["scale"].astype(np.float32), zp, ref)
    # a scale off by more than the tolerance
    s_bad = ref["scale"].astype(np.float32).copy()
    s_bad[2, 1] *= 1.00001
    with pytest.raises(AssertionError):
        check_asym(packed, s_bad, ref["zp"], ref)
