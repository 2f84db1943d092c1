"""Plain float64 CPU oracle for the rotate -> INT4 quantize -> integer GEMM path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path never
calls it, and it shares no code, table or constant with the HIP library.

It is slow on purpose: the Hadamard matrix is built explicitly and applied as
a dense matrix product, quantization is written out element-wise with numpy,
and the integer GEMM is a float64 BLAS product of integer-valued matrices
(exact, see `int_gemm`).

Pages cited (titles; the section follows the dash):
  [ROT]  "Rotations for 4-Bit Activations: QuaRot, SpinQuant, and Friends"
  [QR]   "QuaRot (rotation-based outlier removal, W4A4KV4)" record
  [SQ]   "SpinQuant (learned rotations + W4A4KV4)" record

Readings taken where the pages leave a step open (each is repeated in the
function that uses it):
  * Hadamard = Sylvester construction in natural order.  The randomized
    Hadamard of [QR] "Activation scheme" is diag(d) H with a +-1 vector d
    that the caller draws and passes in (`signs`); None means d = 1.
  * Rotation acts on every row along K, in contiguous aligned blocks of b
    (b = 128 or b = K), i.e. Q = I (x) H_b / sqrt(b).
  * Symmetric INT4: 15 levels -7..7, scale = max|y| / 7, no clipping.
  * Asymmetric INT4: 16 levels 0..15, range widened to include 0,
    zero-point = round(-lo/s), code = round(y/s) + zero-point.
  * Round to nearest, ties to even; an all-zero row or group gets scale 0,
    zero-point 0 and codes 0.
  * Codes are decided from the plain definition in float64 (mode "f64", the
    default): the exact rotated value z, t = 7 z / max|z| (symmetric) or
    t = 15 z / (hi - lo) (asymmetric), rounded to nearest.  The rotation of
    fp16 inputs is exact in float64, so t carries only the rounding of one
    or two float64 operations.
  * A second mode, "f32", evaluates the same formulas in IEEE fp32 with
    correctly rounded division: z rounded once to fp32, the reciprocal
    scale in fp32, their product exact, then rounded to the nearest
    integer.  It exists for inputs whose fp32 rotation is exact (integer
    fp16 values of moderate size), where a GPU that follows that fp32
    formula must reproduce its codes and scales bit for bit.  Outside that
    class the two modes differ only within a few fp32 ulps of a .5 tie.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64


# --------------------------------------------------------------------------
# Hadamard matrix and rotation
# --------------------------------------------------------------------------
def hadamard(n: int) -> np.ndarray:
    """Unnormalized Sylvester Hadamard matrix H_n (int64, entries +-1).

    [ROT] "A rotation changes nothing, and that is the point": Q is a Hadamard
    matrix scaled by 1/sqrt(n), so each entry of Q is +-1/sqrt(n).  The pages
    do not say which Hadamard; the reading is Sylvester's doubling
    H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]], natural order.
    """
    if n < 1 or n & (n - 1):
        raise ValueError(f"Hadamard order must be a power of two, got {n}")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def apply_signs(x, signs) -> np.ndarray:
    """x . diag(d) in float64: column k of every row times d[k] (+-1).

    [QR] "Activation scheme": QuaRot's rotations are randomized Hadamard
    matrices; [ROT] "The recipe": "random-hadamard" vs the fixed "hadamard".
    Read as Q = diag(d) H / sqrt(b) with d a +-1 vector over all K columns,
    the same for activations and weights (Q stays orthogonal since d*d = 1).
    signs None: no flip.
    """
    x = np.asarray(x, dtype=F64)
    if signs is None:
        return x
    d = np.asarray(signs, dtype=F64).reshape(-1)
    if d.shape[0] != x.shape[-1] or not np.all(np.abs(d) == 1.0):
        raise ValueError("signs must be a +-1 vector with one entry per column")
    return x * d[None, :]


def rotate(x, block: int, signs=None) -> np.ndarray:
    """Unnormalized block rotation z = x . diag(d) . (I (x) H_block) of every row, float64.

    [ROT] "A rotation changes nothing": Y = X W^T = (XQ)(WQ)^T for orthogonal Q.
    [ROT] "Gotchas" (block size): a 128-wide block mixes channels in groups of
    128, a full-size Hadamard mixes all of them; [ROT] "The recipe": fixed,
    non-random Hadamard blocks of 128.  block == K is the full-width rotation.

    For fp16 inputs every partial sum is a multiple of 2^-24 below 2^29, so
    the float64 product is exact whatever order BLAS sums in.
    """
    x = apply_signs(x, signs)
    R, K = x.shape
    if K % block:
        raise ValueError("K must be a multiple of the Hadamard block")
    h = hadamard(block).astype(F64)
    z = x.reshape(R, K // block, block) @ h      # H is symmetric: x.H = (H.x^T)^T
    return z.reshape(R, K)


def rotate_normalized(x, block: int, signs=None) -> np.ndarray:
    """y = x . Q with Q = diag(d) (I (x) H_block) / sqrt(block)  ([ROT] "A rotation changes nothing")."""
    return rotate(x, block, signs) / np.sqrt(block)


# --------------------------------------------------------------------------
# Quantizers
# --------------------------------------------------------------------------
def _rne(t: np.ndarray) -> np.ndarray:
    """Round to nearest integer, ties to even ([ROT] "Gotchas": round to nearest)."""
    return np.rint(t)


def quant_sym_rows(z, block: int, mode: str = "f64") -> dict:
    """Symmetric INT4, one scale per row, on unnormalized rotated rows z.

    [ROT] "What it buys in 4 bits": INT4 with one scale per token for the
    activations and one per output channel for the weights.  The normalized
    rotated row is y = z / sqrt(block) (block = 1: no rotation).
    Reading: 15 levels, s = max|y| / 7, q = round(y / s) clamped to [-7, 7],
    round to nearest with ties to even ([ROT] "Gotchas": round to nearest).

    Since y / s = 7 z / max|z|, the code does not depend on the block; it only
    enters the stored scale:  s = max|z| / (7 sqrt(block)).

    mode "f64" (the definition): a = max|z|, s = a / (7 sqrt(block)),
    t = 7 z / a, q = rne(t), all in float64; a = 0 gives s = 0 and q = 0.
    mode "f32" (exact-fp32 form): a = max|fl32(z)|,
    s = fl32(a / fl32(7 sqrt(block))), inv = fl32(7 / a), t = fl32(z) * inv
    held exactly, q = rne(t).
    Returned `t` is the pre-rounding value of the chosen mode.
    """
    if mode == "f64":
        zz = np.asarray(z, dtype=F64)
        a = np.max(np.abs(zz), axis=1)
        nz = a > 0
        safe = np.where(nz, a, 1.0)
        s = np.where(nz, a / (7.0 * np.sqrt(F64(block))), 0.0)
        t = np.where(nz[:, None], 7.0 * zz / safe[:, None], 0.0)
        q = np.clip(_rne(t), -7, 7).astype(np.int8)
        return dict(codes=q, scale=s, t=t, absmax=a, mode=mode)
    if mode != "f32":
        raise ValueError(mode)
    z32 = np.asarray(z, dtype=F64).astype(F32)
    a = np.max(np.abs(z32), axis=1)                       # fp32, exact
    c = F32(7.0 * np.sqrt(F64(block)))
    nz = a > 0
    safe = np.where(nz, a, F32(1))
    s = np.where(nz, safe / c, F32(0)).astype(F32)         # correctly rounded fp32 division
    inv = np.where(nz, F32(7.0) / safe, F32(0)).astype(F32)
    t = z32.astype(F64) * inv.astype(F64)[:, None]       # product of two fp32: exact in f64
    q = np.clip(_rne(t), -7, 7).astype(np.int8)
    return dict(codes=q, scale=s, inv=inv, t=t, absmax=a, mode=mode)


def quant_asym_groups(z, block: int, group: int = 128, mode: str = "f64") -> dict:
    """Asymmetric INT4 with a zero-point, one (scale, zero-point) per group.

    [SQ] "Activation scheme": per-group asymmetric INT4 for weights,
    activations and KV cache; [QR] "Activation scheme": the KV cache is
    rotated too.  The group width is not on the pages; it is 128 here, the
    same contiguous chunk of K as a Hadamard block.
    Reading: lo = min(min y, 0), hi = max(max y, 0), s = (hi - lo) / 15,
    zp = round(-lo / s) in [0, 15], q = round(y / s) + zp clamped to [0, 15];
    dequantized value s * (q - zp).  As in `quant_sym_rows`, the codes depend
    on z only and sqrt(block) enters the scale alone.

    mode "f64" (the definition): r = hi - lo, s = r / (15 sqrt(block)),
    t = 15 z / r, t_zp = -15 lo / r, all in float64.
    mode "f32": r = fl32(hi - lo), s = fl32(r / fl32(15 sqrt(block))),
    inv = fl32(15 / r), the products -lo*inv and z*inv held exactly.
    Either way zp = clamp(rne(t_zp), 0, 15), q = clamp(rne(t) + zp, 0, 15)
    (the integer add comes after rounding); r = 0 gives s = 0, zp = 0, q = 0.
    """
    if mode == "f64":
        zz = np.asarray(z, dtype=F64)
    elif mode == "f32":
        zz = np.asarray(z, dtype=F64).astype(F32)
    else:
        raise ValueError(mode)
    R, K = zz.shape
    if K % group:
        raise ValueError("K must be a multiple of the group width")
    g = zz.reshape(R, K // group, group)
    lo = np.minimum(g.min(axis=2), 0)
    hi = np.maximum(g.max(axis=2), 0)
    if mode == "f64":
        r = hi - lo
        nz = r > 0
        safe = np.where(nz, r, 1.0)
        s = np.where(nz, r / (15.0 * np.sqrt(F64(block))), 0.0)
        t_zp = np.where(nz, -15.0 * lo / safe, 0.0)
        t = np.where(nz[:, :, None], 15.0 * g / safe[:, :, None], 0.0)
        inv = None
    else:
        r = (hi - lo).astype(F32)                            # correctly rounded fp32 subtraction
        c = F32(15.0 * np.sqrt(F64(block)))
        nz = r > 0
        safe = np.where(nz, r, F32(1))
        s = np.where(nz, safe / c, F32(0)).astype(F32)
        inv = np.where(nz, F32(15.0) / safe, F32(0)).astype(F32)
        t_zp = (-lo).astype(F64) * inv.astype(F64)
        t = g.astype(F64) * inv.astype(F64)[:, :, None]
    zp = np.clip(_rne(t_zp), 0, 15)
    q = np.clip(_rne(t) + zp[:, :, None], 0, 15).astype(np.uint8)
    d = dict(codes=q.reshape(R, K), scale=s, zp=zp.astype(np.uint8),
             t=t.reshape(R, K), t_zp=t_zp, lo=lo, hi=hi, mode=mode)
    if inv is not None:
        d["inv"] = inv
    return d


def dequant_sym_rows(q, s) -> np.ndarray:
    """y_hat = s * q, float64 (the scale already carries 1/sqrt(block))."""
    return np.asarray(q, F64) * np.asarray(s, F64)[:, None]


def dequant_asym_groups(q, s, zp, group: int = 128) -> np.ndarray:
    """y_hat = s * (q - zp) per group, float64."""
    q = np.asarray(q, F64)
    R, K = q.shape
    lv = q.reshape(R, K // group, group) - np.asarray(zp, F64)[:, :, None]
    return (lv * np.asarray(s, F64)[:, :, None]).reshape(R, K)


# --------------------------------------------------------------------------
# Nibble packing
# --------------------------------------------------------------------------
def pack_nibbles(q) -> np.ndarray:
    """Two 4-bit codes per byte, even K index in bits 3:0, odd in bits 7:4.

    Signed codes are stored as 4-bit two's complement (-7 -> 0x9), unsigned
    codes as is.  The layout is a reading; the pages only say INT4.
    """
    q = np.asarray(q, dtype=np.int64)
    if q.shape[1] % 2:
        raise ValueError("K must be even to pack nibbles")
    lo = q[:, 0::2] & 0xF
    hi = q[:, 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(p, signed: bool) -> np.ndarray:
    p = np.asarray(p, dtype=np.int64)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    if signed:
        lo = np.where(lo >= 8, lo - 16, lo)
        hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((p.shape[0], 2 * p.shape[1]), dtype=np.int64)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


# --------------------------------------------------------------------------
# Integer GEMM and dequantization epilogues
# --------------------------------------------------------------------------
def int_gemm(qa, qb) -> np.ndarray:
    """acc[m, n] = sum_k qa[m, k] * qb[n, k], exact, int64.

    [ROT] "A rotation changes nothing": the layer computes X W^T; on codes it
    is an integer product.  Evaluated as a float64 BLAS product of
    integer-valued matrices: every term and partial sum is an integer of
    magnitude <= 15 * 7 * K < 2^53, so any summation order is exact.
    """
    qa = np.asarray(qa, dtype=F64)
    qb = np.asarray(qb, dtype=F64)
    bound = np.abs(qa).max(initial=0) * np.abs(qb).max(initial=0) * qa.shape[1]
    if bound >= 2.0 ** 52:
        raise ValueError("integer GEMM would not be exact in float64")
    return np.rint(qa @ qb.T).astype(np.int64)


def epilogue_sym_f32(acc, sx, sw) -> np.ndarray:
    """Y = fl32( fl32(sx[m] * sw[n]) * fl32(acc) ), the fp32 form of Y = s_x s_w acc.

    [ROT] "What it buys in 4 bits": per-token times per-output-channel scales.
    Every fp32 product is correctly rounded; |acc| < 2^24 so fl32(acc) = acc.
    """
    sx = np.asarray(sx, F32)
    sw = np.asarray(sw, F32)
    ss = (sx[:, None] * sw[None, :]).astype(F32)
    return (ss * np.asarray(acc, F64).astype(F32)).astype(F32)


def epilogue_sym_f64(acc, sx, sw) -> np.ndarray:
    return np.asarray(sx, F64)[:, None] * np.asarray(sw, F64)[None, :] * np.asarray(acc, F64)


def group_sums(qw, group: int = 128) -> np.ndarray:
    """gsum[n, g] = sum of weight codes of row n over K-group g (int64)."""
    qw = np.asarray(qw, dtype=np.int64)
    N, K = qw.shape
    return qw.reshape(N, K // group, group).sum(axis=2)


def gemm_asym_f64(u, zp, sx, qw, sw, group: int = 128) -> np.ndarray:
    """Y[m, n] = sw[n] * sum_g sx[m, g] * sum_{k in g} (u[m, k] - zp[m, g]) * qw[n, k].

    Asymmetric per-group activations ([SQ] "Activation scheme") against
    symmetric per-channel weights; each group's integer dot product of the
    activation levels with the weight codes is exact, then scaled in float64.
    """
    u = np.asarray(u, F64)
    M, K = u.shape
    G = K // group
    lv = u.reshape(M, G, group) - np.asarray(zp, F64)[:, :, None]
    qw = np.asarray(qw, F64).reshape(-1, G, group)
    y = np.zeros((M, qw.shape[0]), dtype=F64)
    for g in range(G):
        Ag = np.rint(lv[:, g, :] @ qw[:, g, :].T)          # exact integers
        y += np.asarray(sx, F64)[:, g][:, None] * Ag
    return y * np.asarray(sw, F64)[None, :]


def int_gemm_groups(u, zp, qw, group: int = 128) -> np.ndarray:
    """A'[m, n, g] = sum_{k in g} (u[m, k] - zp[m, g]) * qw[n, k], exact int64."""
    u = np.asarray(u, F64)
    M, K = u.shape
    G = K // group
    lv = u.reshape(M, G, group) - np.asarray(zp, F64)[:, :, None]
    qw = np.asarray(qw, F64).reshape(-1, G, group)
    return np.rint(np.einsum("mgk,ngk->mng", lv, qw)).astype(np.int64)


# --------------------------------------------------------------------------
# End-to-end pieces of the path
# --------------------------------------------------------------------------
def rotate_quant_act(x, block: int, mode: str, signs=None, decide: str = "f64") -> dict:
    """Online activation step: rotate each token, quantize, pack.

    [ROT] "Where the rotations go": rotations that cannot be folded into the
    weights cost one fast Hadamard transform per token, fused with the
    quantization of the activations.  mode "sym": one scale per token;
    mode "asym": asymmetric per group of 128 with a zero-point.  signs: the
    randomized-Hadamard diagonal (see `apply_signs`), or None.  decide: the
    quantizer's arithmetic, "f64" (the definition) or "f32" (exact-fp32 form).
    """
    z = rotate(x, block, signs)
    if mode == "sym":
        d = quant_sym_rows(z, block, decide)
        d["packed"] = pack_nibbles(d["codes"])
    elif mode == "asym":
        d = quant_asym_groups(z, block, 128, decide)
        d["packed"] = pack_nibbles(d["codes"])
    else:
        raise ValueError(mode)
    d["z"] = z
    return d


def quant_weight_offline(w, block: int, signs=None, decide: str = "f64") -> dict:
    """Offline weight step: rotate each output channel's row, symmetric INT4
    per output channel, pack, and the per-128 group sums of the codes.

    [ROT] "Where the rotations go": rotations applied to weights are folded
    offline and cost nothing at run time.  signs: the same diagonal the
    activations use, or None.  decide: as in `rotate_quant_act`.
    """
    z = rotate(w, block, signs)
    d = quant_sym_rows(z, block, decide)
    d["packed"] = pack_nibbles(d["codes"])
    d["gsum"] = group_sums(d["codes"], 128)
    d["z"] = z
    return d


def w4a4_linear(x, w, block: int, mode: str = "sym", signs=None, decide: str = "f64") -> dict:
    """Y_hat = Q(XQ) . Q(WQ)^T and the float64 X W^T it approximates.

    [ROT] "A rotation changes nothing" (invariance) and "What it buys in 4
    bits" (the quantized product).
    """
    a = rotate_quant_act(x, block, mode, signs, decide)
    wq = quant_weight_offline(w, block, signs, decide)
    if mode == "sym":
        acc = int_gemm(a["codes"], wq["codes"])
        y = epilogue_sym_f64(acc, a["scale"], wq["scale"])
    else:
        acc = None
        y = gemm_asym_f64(a["codes"], a["zp"], a["scale"], wq["codes"], wq["scale"])
    return dict(act=a, wq=wq, acc=acc, y=y)


def kv_rotate_quant(kv, block: int = 128, signs=None, decide: str = "f64") -> dict:
    """KV cache step: rotate every (batch, head, token) vector of head_dim 128
    with one 128-point Hadamard, then asymmetric INT4 with a zero-point, one
    group per vector.

    [QR] "Activation scheme": the KV cache is rotated as well;
    [SQ] "Activation scheme": per-group asymmetric INT4 on the KV cache.
    decide: as in `rotate_quant_act`.
    """
    kv = np.asarray(kv)
    shape = kv.shape
    D = shape[-1]
    flat = kv.reshape(-1, D)
    z = rotate(flat, block, signs)
    d = quant_asym_groups(z, block, D, decide)
    d["packed"] = pack_nibbles(d["codes"]).reshape(*shape[:-1], D // 2)
    d["scale"] = d["scale"].reshape(shape[:-1])
    d["zp"] = d["zp"].reshape(shape[:-1])
    d["z"] = z
    return d


# --------------------------------------------------------------------------
# MXFP4: E2M1 elements with a power-of-two scale shared by 32 values
# --------------------------------------------------------------------------
# [ROT] "The full model in NVFP4, on vLLM" / "When to rotate": MXFP4 is a 4-bit format whose scales
# are powers of two shared by 32 values, and rotations help it (unlike
# NVFP4).  Reading (the pages give no formulas; this is the usual MX
# convention): the element grid is E2M1, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}
# for codes 0..7 with bit 3 the sign; the shared scale of a block is
# 2^e, e = floor(log2(max|y|)) - 2 (2 = the exponent of E2M1's largest value),
# stored as the biased byte e + 127; elements round to nearest on the grid,
# ties to the even code, and saturate at +-6.  A block of zeros gets the
# byte 0 and zero codes.  What is quantized is the normalized rotated value
# y = x Q = z / sqrt(b) (the scale is a power of two, so 1/sqrt(b) matters
# here), in float64; the exact-fp32 form y = fl32(fl32(z) * fl32(1/sqrt(b)))
# is the second mode, for inputs whose fp32 rotation is exact.
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MX_BLOCK = 32


def e2m1_value(codes) -> np.ndarray:
    """Decode 4-bit E2M1 codes (bit 3 = sign) to float64."""
    c = np.asarray(codes, dtype=np.int64)
    mag = E2M1[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_round(t) -> np.ndarray:
    """Nearest E2M1 code of each value (ties to the even code, saturating at 6).

    Written out as the distance to every grid point; among equally near
    points the one with an even code wins.
    """
    t = np.asarray(t, dtype=F64)
    a = np.minimum(np.abs(t), 6.0)
    d = np.abs(a[..., None] - E2M1)                        # distance to each magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # prefer the even code among the nearest (codes are 0..7 in grid order)
    even = cand & ((np.arange(8) % 2) == 0)
    pick = np.where(even.any(axis=-1, keepdims=True), even, cand)
    mag = np.argmax(pick, axis=-1)
    neg = (t < 0) & (mag > 0)
    return (mag + 8 * neg).astype(np.int64)


def mx_quant_rows(y, block: int = MX_BLOCK) -> dict:
    """MXFP4 quantization of rows y [R, K] (float64 values) in blocks of 32 along K.

    Returns codes [R, K] (0..15), scale_e [R, K/32] (the exponent e) and
    scale_byte (e + 127).
    """
    y = np.asarray(y, dtype=F64)
    R, K = y.shape
    yb = y.reshape(R, K // block, block)
    amax = np.abs(yb).max(axis=-1)
    mant, ex = np.frexp(amax)                              # amax = mant * 2^ex, mant in [0.5, 1)
    e = np.where(amax > 0, ex - 1 - 2, -127)               # floor(log2 amax) - 2
    e = np.clip(e, -127, 127).astype(np.int64)
    t = yb / np.exp2(e.astype(F64))[..., None]             # exact: division by a power of two
    codes = e2m1_round(t).reshape(R, K)
    return dict(codes=codes, scale_e=e, scale_byte=(e + 127).astype(np.uint8))


def mx_dequant_rows(codes, scale_e, block: int = MX_BLOCK) -> np.ndarray:
    c = np.asarray(codes)
    R, K = c.shape
    v = e2m1_value(c).reshape(R, K // block, block)
    return (v * np.exp2(np.asarray(scale_e, dtype=F64))[..., None]).reshape(R, K)


def rotate_mx_quant(x, block: int, signs=None, decide: str = "f64") -> dict:
    """Rotate each row (Q = diag(d) H_block / sqrt(block)), then MXFP4.

    [ROT] "The full model in NVFP4, on vLLM" and "When to rotate": rotations
    help MXFP4, whose scales are powers of two shared by 32 values.  Codes
    are packed two per byte like the INT4 codes.
    decide "f64": y = z / sqrt(block) in float64 (the definition);
    "f32": y = fl32(fl32(z) * fl32(1 / sqrt(block))).  Returned `y` is the
    value that was quantized.
    """
    z = rotate(x, block, signs)
    if decide == "f64":
        y = z / np.sqrt(F64(block))
    elif decide == "f32":
        y = (z.astype(F32) * F32(1.0 / np.sqrt(block))).astype(F32).astype(F64)
    else:
        raise ValueError(decide)
    d = mx_quant_rows(y)
    d["packed"] = pack_nibbles(d["codes"])
    d["y"] = y
    d["mode"] = decide
    return d


def mx_gemm_f64(ca, ea, cb, eb, block: int = MX_BLOCK) -> np.ndarray:
    """Y[m, n] = sum over 32-blocks j of 2^(ea[m,j] + eb[n,j]) * sum_{k in j} a[m,k] b[n,k],
    in float64 (every term is a dyadic rational; exact for these sizes)."""
    va = e2m1_value(ca)
    vb = e2m1_value(cb)
    M, K = va.shape
    N = vb.shape[0]
    J = K // block
    part = np.einsum("mjk,njk->mnj", va.reshape(M, J, block), vb.reshape(N, J, block))
    return np.einsum("mnj,mnj->mn", part, np.exp2(np.asarray(ea, F64)[:, None, :] + np.asarray(eb, F64)[None, :, :]))


# --------------------------------------------------------------------------
# Decode attention over the rotated INT4 KV cache
# --------------------------------------------------------------------------
def attention_decode_f64(q, k, v, softmax_scale: float) -> np.ndarray:
    """Textbook single-query attention per (batch, head), float64:
    o = sum_t p_t v_t with p = softmax_t(softmax_scale * q . k_t).

    q [B, H, D], k and v [B, H, S, D]; returns o [B, H, D].
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    scores = softmax_scale * np.einsum("bhd,bhsd->bhs", q, k)
    scores -= scores.max(axis=-1, keepdims=True)
    p = np.exp(scores)
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("bhs,bhsd->bhd", p, v)


def kv4_attention_decode(q, k_packed, k_scale, k_zp, v_packed, v_scale, v_zp,
                         softmax_scale: float, signs=None) -> np.ndarray:
    """Single-query attention over a KV cache stored as rotated asymmetric INT4.

    [QR] "Activation scheme": the KV cache and parts of the attention
    computation are rotated; [ROT] "A rotation changes nothing": with an
    orthogonal Q, (q Q) . (k Q) = q . k, so scores can be taken between the
    rotated query and the rotated keys, and the weighted sum of rotated values
    is rotated back once: o = o_rot Q^T.  Here Q = diag(d) H_D / sqrt(D)
    (d = 1 without signs), the same Q the KV step used.

    k_packed/v_packed [B, H, S, D/2] unsigned nibbles; k_scale/v_scale and
    k_zp/v_zp [B, H, S] (one group per head vector); the dequantized rotated
    vectors are scale * (code - zp) (see `dequant_asym_groups`).
    Returns o [B, H, D] float64.
    """
    q = np.asarray(q, dtype=F64)
    B, H, D = q.shape
    S = np.asarray(k_packed).shape[2]

    def deq(packed, scale, zp):
        u = unpack_nibbles(np.asarray(packed).reshape(-1, D // 2), signed=False)
        flat = dequant_asym_groups(u, np.asarray(scale).reshape(-1, 1), np.asarray(zp).reshape(-1, 1), D)
        return flat.reshape(B, H, S, D)

    q_rot = rotate_normalized(q.reshape(-1, D), D, signs).reshape(B, H, D)
    o_rot = attention_decode_f64(q_rot, deq(k_packed, k_scale, k_zp), deq(v_packed, v_scale, v_zp),
                                 softmax_scale)
    # o = o_rot Q^T = o_rot H diag(d) / sqrt(D)   (H symmetric)
    h = hadamard(D).astype(F64)
    o = (o_rot.reshape(-1, D) @ h) / np.sqrt(D)
    o = apply_signs(o, signs)
    return o.reshape(B, H, D)


# --------------------------------------------------------------------------
# Statistics the rotation page measures
# --------------------------------------------------------------------------
def kurtosis(v) -> float:
    """Pearson kurtosis E[(v-mu)^4] / E[(v-mu)^2]^2 over all elements.

    [ROT] "A rotation changes nothing": 3 for a Gaussian, hundreds to
    thousands when a few channels dominate (so Pearson, not excess).
    """
    v = np.asarray(v, dtype=F64).ravel()
    d = v - v.mean()
    m2 = np.mean(d * d)
    return float(np.mean(d ** 4) / (m2 * m2))


def outlier_ratio(x) -> float:
    """Largest |value| over the median, across channels, of each channel's
    largest |value| over tokens ([ROT] "A rotation changes nothing")."""
    a = np.abs(np.asarray(x, dtype=F64))
    return float(a.max() / np.median(a.max(axis=0)))


def product_error(x, w, x_hat, w_hat) -> float:
    """||X W^T - X_hat W_hat^T||_F / ||X W^T||_F  ([ROT] "What it buys in 4 bits")."""
    ref = np.asarray(x, F64) @ np.asarray(w, F64).T
    got = np.asarray(x_hat, F64) @ np.asarray(w_hat, F64).T
    return float(np.linalg.norm(ref - got) / np.linalg.norm(ref))
