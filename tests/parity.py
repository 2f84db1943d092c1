"""GPU-vs-oracle comparison rules (test helper).

Codes may differ from the oracle's only where the oracle's pre-rounding value
t lies within TIE_WINDOW of a .5 tie (the GPU transform runs in fp32, the
oracle's exactly), by one level, and at most MAX_FLIP_FRAC of the elements.
Packed bytes must agree wherever both of their codes agree.  Scales agree to
SCALE_RTOL relative (bit-exact on the exact-arithmetic inputs).
"""
from __future__ import annotations

import numpy as np

import oracle as O

TIE_WINDOW = 1e-5
MAX_FLIP_FRAC = 1e-4
SCALE_RTOL = 1e-6
Y_RTOL_FRO = 1e-3


def near_tie(t: np.ndarray) -> np.ndarray:
    return np.abs(np.abs(t - np.floor(t)) - 0.5) < TIE_WINDOW


def ulp_diff(a: np.ndarray, b: np.ndarray) -> int:
    a = np.ascontiguousarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.ascontiguousarray(b, np.float32).view(np.int32).astype(np.int64)
    return int(np.abs(a - b).max(initial=0))


def check_sym(packed_gpu, scales_gpu, ref: dict, exact: bool = False) -> dict:
    """Compare GPU symmetric codes/scales with oracle `quant_sym_rows` output."""
    q_gpu = O.unpack_nibbles(packed_gpu, signed=True)
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
    """Compare GPU asymmetric codes/scales/zero-points with `quant_asym_groups` output."""
    R = ref["codes"].shape[0]
    G = ref["zp"].shape[1]
    u_gpu = O.unpack_nibbles(packed_gpu.reshape(R, -1), signed=False)
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
