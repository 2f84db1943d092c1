"""GPU-vs-oracle comparison rules (test helper).

Codes may differ from the oracle's only where the oracle's float64
pre-rounding value t (the plain definition, t = 7 z / max|z| or 15 z / r)
lies within TIE_WINDOW of a .5 tie (the GPU transform runs in fp32, the
oracle's exactly), by one level, and at most MAX_FLIP_FRAC of the elements.
Packed bytes must agree wherever both of their codes agree.  Scales agree to
SCALE_RTOL relative.  On the exact-arithmetic inputs the GPU must instead
equal the oracle's exact-fp32 mode bit for bit (codes, scales, bytes).
"""
from __future__ import annotations

import numpy as np

import oracle as O

TIE_WINDOW = 1e-5
MAX_FLIP_FRAC = 1e-4
SCALE_RTOL = 1e-6
Y_RTOL_FRO = 1e-3


def decode_nibbles(packed, signed: bool) -> np.ndarray:
    """The packed code layout read back on the test side (even index in bits
    3:0, odd index in bits 7:4, signed codes in two's complement), so that GPU
    output is decoded without the oracle's own helpers."""
    p = np.asarray(packed, np.uint8)
    p = p.reshape(p.shape[0], -1)
    u = np.empty((p.shape[0], 2 * p.shape[1]), np.int64)
    u[:, 0::2] = p & 0xF
    u[:, 1::2] = p >> 4
    return np.where(u >= 8, u - 16, u) if signed else u


def nibble_group_sums(packed, group: int = 128) -> np.ndarray:
    """Per-group sums of the signed codes held in `packed` (test side)."""
    q = decode_nibbles(packed, signed=True)
    return q.reshape(q.shape[0], -1, group).sum(axis=-1)


def check_gsum(gsum_gpu, packed_gpu, ref: dict) -> None:
    """Group sums: the sums of the codes the GPU wrote on every row, and the
    oracle's own sums on every row whose codes equal the oracle's."""
    g = np.asarray(gsum_gpu, np.int64)
    assert np.array_equal(g, nibble_group_sums(packed_gpu)), "group sums are not the sums of the codes"
    same = np.all(decode_nibbles(packed_gpu, signed=True) == ref["codes"], axis=1)
    assert np.array_equal(g[same], np.asarray(ref["gsum"], np.int64)[same])


def near_tie(t: np.ndarray) -> np.ndarray:
    return np.abs(np.abs(t - np.floor(t)) - 0.5) < TIE_WINDOW


def ulp_diff(a: np.ndarray, b: np.ndarray) -> int:
    a = np.ascontiguousarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.ascontiguousarray(b, np.float32).view(np.int32).astype(np.int64)
    return int(np.abs(a - b).max(initial=0))


def check_sym(packed_gpu, scales_gpu, ref: dict, exact: bool = False) -> dict:
    """Compare GPU symmetric codes/scales with oracle `quant_sym_rows` output:
    the float64 mode under the tie rule, or (exact=True) the exact-fp32 mode
    bit for bit."""
    assert ref["mode"] == ("f32" if exact else "f64"), "wrong oracle mode for this comparison"
    q_gpu = decode_nibbles(packed_gpu, signed=True)
    q_ref = ref["codes"].astype(np.int64)
    assert q_gpu.shape == q_ref.shape
    diff = q_gpu != q_ref
    n_flip = int(diff.sum())
    if exact:
        assert n_flip == 0, f"{n_flip} code mismatches on exact inputs"
        assert np.array_equal(np.asarray(scales_gpu, np.float32), ref["scale"])
    else:
        assert np.all(np.abs(q_gpu - q_ref)[diff] == 1), "a code differs by more than one level"
        assert np.all(near_tie(ref["t"][diff])), "a code differs away from a rounding tie"
        assert n_flip <= MAX_FLIP_FRAC * q_ref.size, f"{n_flip} flips in {q_ref.size}"
        s_ref = ref["scale"].astype(np.float64)
        s_gpu = np.asarray(scales_gpu, np.float64)
        assert np.all(np.abs(s_gpu - s_ref) <= SCALE_RTOL * np.abs(s_ref)), "scale mismatch"
    _check_bytes(packed_gpu, q_ref, diff)
    return dict(flips=n_flip, elements=q_ref.size, scale_ulp=ulp_diff(scales_gpu, ref["scale"]))


def check_asym(packed_gpu, scales_gpu, zeros_gpu, ref: dict, exact: bool = False) -> dict:
    """Compare GPU asymmetric codes/scales/zero-points with `quant_asym_groups`
    output (float64 mode under the tie rule, or exact-fp32 mode bit for bit)."""
    assert ref["mode"] == ("f32" if exact else "f64"), "wrong oracle mode for this comparison"
    R = ref["codes"].shape[0]
    G = ref["zp"].shape[1]
    u_gpu = decode_nibbles(np.asarray(packed_gpu).reshape(R, -1), signed=False)
    zp_gpu = np.asarray(zeros_gpu).reshape(R, G).astype(np.int64)
    zp_ref = ref["zp"].astype(np.int64)
    s_gpu = np.asarray(scales_gpu, np.float32).reshape(R, G)
    zdiff = zp_gpu != zp_ref
    if exact:
        assert not zdiff.any()
        assert np.array_equal(u_gpu, ref["codes"].astype(np.int64))
        assert np.array_equal(s_gpu, ref["scale"])
        return dict(flips=0, zp_flips=0, elements=u_gpu.size, scale_ulp=0)
    assert np.all(near_tie(ref["t_zp"][zdiff])), "a zero-point differs away from a tie"
    assert np.all(np.abs(zp_gpu - zp_ref)[zdiff] == 1)
    # levels (code - zero) are what the dequantized value depends on; compare those
    lv_gpu = u_gpu.reshape(R, G, -1) - zp_gpu[:, :, None]
    lv_ref = ref["codes"].astype(np.int64).reshape(R, G, -1) - zp_ref[:, :, None]
    diff = lv_gpu != lv_ref
    t = ref["t"].reshape(R, G, -1)
    zt = np.broadcast_to(ref["t_zp"][:, :, None], t.shape)
    ok_elem = near_tie(t) | near_tie(zt)      # a zero-point tie shifts the whole group
    assert np.all(ok_elem[diff]), "a level differs away from a rounding tie"
    n_flip = int(diff.sum())
    assert n_flip <= MAX_FLIP_FRAC * lv_ref.size + 128 * int(zdiff.sum()), f"{n_flip} flips"
    s_ref = ref["scale"].astype(np.float64)
    assert np.all(np.abs(s_gpu - s_ref) <= SCALE_RTOL * np.abs(s_ref)), "scale mismatch"
    same = ~diff.reshape(R, -1) & np.repeat(~zdiff, u_gpu.shape[1] // G, axis=1)
    _check_bytes(packed_gpu.reshape(R, -1), ref["codes"].astype(np.int64), ~same)
    return dict(flips=n_flip, zp_flips=int(zdiff.sum()), elements=lv_ref.size,
                scale_ulp=ulp_diff(s_gpu, ref["scale"]))


def _check_bytes(packed_gpu, q_ref, diff):
    p_ref = O.pack_nibbles(q_ref)
    both_ok = ~(diff[:, 0::2] | diff[:, 1::2])
    pg = np.asarray(packed_gpu).reshape(p_ref.shape)
    assert np.array_equal(pg[both_ok], p_ref[both_ok]), "packed bytes differ where codes agree"


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ---------------------------------------------------------------- MXFP4
E2M1_TIES = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def near_mx_tie(t: np.ndarray) -> np.ndarray:
    """|t| within TIE_WINDOW (relative to the tie, at least absolute) of a
    midpoint between two E2M1 magnitudes."""
    a = np.abs(np.asarray(t, np.float64))
    d = np.abs(a[..., None] - E2M1_TIES)
    return (d < TIE_WINDOW * np.maximum(1.0, E2M1_TIES)).any(axis=-1)


def check_mx(packed_gpu, sbytes_gpu, ref: dict, exact: bool = False) -> dict:
    """Compare GPU MXFP4 codes / scale bytes with oracle `rotate_mx_quant` output.

    An exponent may differ (by one) only where the oracle's block maximum is
    within TIE_WINDOW of a power of two; such a block's codes are checked
    against the oracle's rounding of y under that neighbouring exponent.
    Codes may differ (by one
    magnitude step) only near an E2M1 midpoint.  `ref` is the float64 mode,
    or (exact=True) the exact-fp32 mode, which must match bit for bit."""
    assert ref["mode"] == ("f32" if exact else "f64"), "wrong oracle mode for this comparison"
    y = np.asarray(ref["y"], np.float64)
    R, K = y.shape
    J = K // 32
    e_ref = np.asarray(ref["scale_e"], np.int64)
    e_gpu = np.asarray(sbytes_gpu, np.int64).reshape(R, J) - 127
    ediff = e_gpu != e_ref
    if exact:
        assert not ediff.any(), f"{int(ediff.sum())} exponent mismatches on exact inputs"
    else:
        amax = np.abs(y.reshape(R, J, 32)).max(axis=-1)
        pos = amax > 0
        mant = np.where(pos, amax / np.exp2(np.floor(np.log2(np.where(pos, amax, 1.0)))), 1.5)
        near_p2 = (np.abs(mant - 1.0) < TIE_WINDOW) | (np.abs(mant - 2.0) < TIE_WINDOW)
        assert np.all(near_p2[ediff]), "an exponent differs away from a power of two"
        assert np.all(np.abs(e_gpu - e_ref)[ediff] == 1)
    # expected codes: the oracle's, or, in a block whose exponent legitimately
    # moved by one, the oracle's rounding of y under that neighbouring exponent
    t_ref = y.reshape(R, J, 32) / np.exp2(e_ref.astype(np.float64))[..., None]
    c_exp = np.asarray(ref["codes"], np.int64).reshape(R, J, 32)
    for step in (-1, 1):
        sel = (e_gpu - e_ref) == step
        if sel.any():
            c_alt = O.e2m1_round(t_ref[sel] / 2.0 ** step)
            c_exp[sel] = c_alt
    t = t_ref.copy()
    t[ediff] = t_ref[ediff] / np.exp2((e_gpu - e_ref)[ediff].astype(np.float64))[..., None]
    c_exp = c_exp.reshape(R, K)
    c_gpu = decode_nibbles(packed_gpu, signed=False).reshape(R, K)
    diff = c_gpu != c_exp
    n_flip = int(diff.sum())
    if exact:
        assert n_flip == 0, f"{n_flip} code mismatches on exact inputs"
    else:
        mg, me = c_gpu & 7, c_exp & 7
        assert np.all(np.abs(mg - me)[diff] == 1), "a code differs by more than one step"
        same_sign = ((c_gpu ^ c_exp) & 8) == 0
        assert np.all((same_sign | (mg == 0) | (me == 0))[diff]), "a code differs in sign"
        assert np.all(near_mx_tie(t.reshape(R, K)[diff])), "a code differs away from a midpoint"
        assert n_flip <= MAX_FLIP_FRAC * c_exp.size, f"{n_flip} flips in {c_exp.size}"
    _check_bytes(np.asarray(packed_gpu).reshape(R, -1), c_exp, diff)
    return dict(flips=n_flip, scale_flips=int(ediff.sum()), elements=c_exp.size)
