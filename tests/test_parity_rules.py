"""The GPU-vs-oracle comparison rules themselves (CPU): they accept the
oracle's own output and reject planted mistakes of the kinds a kernel could
make (a wrong code away from a tie, a wrong exponent, swapped nibbles)."""
import numpy as np
import pytest

import oracle as O
import workloads as WL
from parity import check_mx, check_sym, near_mx_tie


@pytest.fixture(scope="module")
def mx_ref():
    x = WL.small_random(404, 24, 512, outlier_cols=[5, 300], mult=30.0)
    return O.rotate_mx_quant(x, 128)


def test_check_mx_accepts_the_oracle(mx_ref):
    st = check_mx(mx_ref["packed"], mx_ref["scale_byte"], mx_ref, exact=True)
    assert st["flips"] == 0 and st["scale_flips"] == 0


def test_check_mx_rejects_a_code_away_from_a_midpoint(mx_ref):
    c = mx_ref["codes"].copy()
    t = mx_ref["y32"].reshape(c.shape[0], -1, 32) / np.exp2(mx_ref["scale_e"])[..., None]
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
    check_sym(packed, ref["scale"], ref, exact=True)
    c = ref["codes"].astype(np.int64).copy()
    far = np.abs(np.abs(ref["t"] - np.floor(ref["t"])) - 0.5) > 0.1
    i, j = np.argwhere(far & (np.abs(c) < 7))[0]
    c[i, j] += 1
    with pytest.raises(AssertionError):
        check_sym(O.pack_nibbles(c), ref["scale"], ref)
