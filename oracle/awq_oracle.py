"""CPU oracle for the AWQ per-layer search path and for inference with its
packed output -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's smoke check and the benchmark's CPU
baseline leg may import this module.  The product path never calls it: it is
the plain, slow, obviously correct statement of what the GPU path computes,
written from the pages and sharing no code with the HIP kernels.

Sources (cited by page title and section):
  [P1] dev.to, "AWQ: How Activation-Aware Quantization Saves 4-bit LLMs"
       - "How does AWQ decide which weights to protect?" (channel_importance listing)
       - "How does AWQ protect channels without mixed precision?" (search_scale listing)
       - "What do you actually deploy" (quant_config: zero point, group 128, 4 bit)
  [P2] esaholic.com, "What is AWQ Quantization?", pipeline step
       "INT4 Weight Packing & Export" (codes packed into INT32 containers)
  [P3] modelrefs.com, "AWQ (Activation-Aware Weight Quantization) -- AI Glossary",
       "Example: Where 4-bit memory saving comes from"
  [P4] mbrenndoerfer.com, "AWQ > Salient Weight Preservation",
       step-size equation s_q = (w_max - w_min)/(2^b - 1) and the scaling identity
  [P5] mbrenndoerfer.com, "AWQ > Summary", "Salient weight identification",
       "The scaling formula"

Precision (the pages fix none of it, so these are readings):
  * element-wise quantizer arithmetic is IEEE binary32 with round-to-nearest-
    even, as numpy float32 performs it: the integer codes are decided in the
    same precision the kernels use;
  * sums and contractions are binary64 (exact products of fp16 inputs);
  * the dequantized weight is rounded once to fp16 from the exact product of
    the binary32 value (q - z) * step and the binary32 reciprocal of s.

Every function here is pinned by tests that do not re-use its own formulas:
worked examples built on the quantization grid, exact rational brute force,
closed forms on Hadamard inputs, invariances and the page's memory
arithmetic.  The one result with no external pin is the absolute value of the
losses on the large synthetic configurations (parity there is GPU vs. this
oracle only).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

F16, F32, F64 = np.float16, np.float32, np.float64

#: default search settings: quant_config of [P1] "What do you actually deploy"
#: (zero point on, group 128, 4 bit) and the grid size and floor of the
#: search_scale listing in [P1] "How does AWQ protect channels".
W_BIT = 4
GROUP = 128
N_GRID = 20
SAL_FLOOR = F32(1e-4)


class NonFiniteLosses(ArithmeticError):
    """No grid point produced a finite loss (the listing then keeps no scale)."""


# --------------------------------------------------------------------------
# step 1: activation saliency
# --------------------------------------------------------------------------
def act_stats(X: np.ndarray) -> np.ndarray:
    """Per-input-channel saliency: the mean of |X[t, k]| over calibration tokens.

    [P1] channel_importance listing (abs, then mean over the token axis);
    [P5] "Salient weight identification" (average absolute activation).

    The sum is exact: |x| of a finite fp16 value is an integer multiple of
    2^-24, so summing those integers is exact for any token count.  The mean
    is then the binary64 quotient, rounded to binary32.

    Non-finite inputs follow IEEE addition of the |x| values: a channel with
    a NaN has saliency NaN, otherwise a channel with an infinity has +inf.
    """
    X = np.asarray(X)
    if X.dtype != F16 or X.ndim != 2:
        raise TypeError("X must be a 2-D float16 array [tokens, in_features]")
    n = X.shape[0]
    a = np.abs(X).astype(F64)
    finite = np.isfinite(a)
    units = (np.where(finite, a, 0.0) * 2.0 ** 24).astype(np.int64)  # exact integers
    total = units.sum(axis=0, dtype=np.int64)                        # exact
    mean = (total.astype(F64) * 2.0 ** -24 / F64(n)).astype(F32)
    has_inf = np.isinf(a).any(axis=0)
    has_nan = np.isnan(a).any(axis=0)
    mean = np.where(has_inf, F32(np.inf), mean)
    return np.where(has_nan, F32(np.nan), mean).astype(F32)


# --------------------------------------------------------------------------
# step 2: per-channel scales for every grid point
# --------------------------------------------------------------------------
def alphas(n_grid: int = N_GRID) -> np.ndarray:
    """alpha_i = i / n_grid for i = 0 .. n_grid-1 ([P1] search_scale listing:
    0 means no scaling; the grid stops one point short of 1)."""
    return np.arange(n_grid, dtype=F64) / F64(n_grid)


def scale_table(sal: np.ndarray, n_grid: int = N_GRID, floor: float = SAL_FLOOR):
    """s[i, k] = max(sal_k, floor) ** alpha_i and its reciprocal.

    [P1] search_scale listing: the saliency is clamped from below at 1e-4 and
    raised to alpha; [P5] "The scaling formula".  The power is taken in
    binary64 and rounded to binary32; the reciprocal is a binary32 division.
    """
    sal = np.asarray(sal, dtype=F32)
    base = np.maximum(sal, F32(floor)).astype(F64)
    s = np.power(base[None, :], alphas(n_grid)[:, None]).astype(F32)
    inv_s = (F32(1.0) / s).astype(F32)
    return s, inv_s


# --------------------------------------------------------------------------
# step 3: asymmetric group quantization of W * diag(s)
# --------------------------------------------------------------------------
@dataclass
class GroupQuant:
    step: np.ndarray   # [rows, n_groups] float32
    zero: np.ndarray   # [rows, n_groups] float32 (an integer value, +0 for zero)
    q: np.ndarray      # [rows, in] uint8 codes in 0 .. 2^b-1
    tie: np.ndarray    # [rows, in] bool: the code's pre-round value, or its
                       # group's zero-point pre-round value, within 1 ulp of a .5 tie
    zero_tie: Optional[np.ndarray] = None  # [rows, n_groups] bool: the zero's pre-round
                                           # value within 1 ulp of a .5 tie


def _near_half(x: np.ndarray) -> np.ndarray:
    """True where the binary32 value x lies within one binary32 ulp of x of a
    half-integer (a value round-half-to-even could send either way once the
    quotient before it is off by an ulp).  Where every binary32 value is an
    integer (|x| >= 2^23) that holds for every x."""
    frac = np.abs(x.astype(F64) - (np.floor(x.astype(F64)) + 0.5))
    return frac <= np.spacing(np.abs(x).astype(F32)).astype(F64)


def quantize(ws: np.ndarray, group: int = GROUP, w_bit: int = W_BIT,
             zero_point: bool = True) -> GroupQuant:
    """Quantize binary32 rows group-wise to w_bit integers.

    Asymmetric (zero_point, the method's setting): [P4] step-size equation,
    step = (max - min) / (2^b - 1) over a group; [P1] quant_config: zero point
    on, groups of 128 along in_features; [P3] "How it works", step 4: every
    group has its own scale.  Per group (binary32, round half to even):
        step = (mx - mn) / (2^b - 1)   (a zero range takes step = 1)
        zero = rint(-mn / step)        (not clamped; -0 becomes +0)
        q    = clamp(rint(w / step) + zero, 0, 2^b - 1)

    Symmetric (the round-to-nearest baseline of [P1] "Why does naive 4-bit
    quantization wreck LLM accuracy?": step = max|w| / 2^(b-1), value
    step * round(w / step)); the rounded value is clamped to the b-bit signed
    range [-2^(b-1), 2^(b-1) - 1] and stored offset by 2^(b-1), i.e. with the
    fixed zero point 2^(b-1), so both variants dequantize as (q - zero) step.
    """
    ws = np.asarray(ws)
    if ws.dtype != F32 or ws.ndim != 2 or ws.shape[1] % group:
        raise TypeError("ws must be float32 [rows, in] with in a multiple of the group")
    rows, k = ws.shape
    qmax = F32(2 ** w_bit - 1)
    g = ws.reshape(rows, k // group, group)
    mn = g.min(axis=2)
    mx = g.max(axis=2)
    if zero_point:
        step = ((mx - mn) / qmax).astype(F32)
        step = np.where(step == F32(0), F32(1), step).astype(F32)
        zpre = (-mn / step).astype(F32)
        zero = (np.rint(zpre) + F32(0)).astype(F32)
    else:
        amax = np.maximum(np.abs(mn), np.abs(mx))
        step = (amax / F32(2 ** (w_bit - 1))).astype(F32)
        step = np.where(step == F32(0), F32(1), step).astype(F32)
        zpre = np.zeros_like(step)
        zero = np.full_like(step, F32(2 ** (w_bit - 1)))
    x = (g / step[:, :, None]).astype(F32)
    q = np.clip(np.rint(x) + zero[:, :, None], F32(0), qmax).astype(F32)
    zero_tie = _near_half(zpre) if zero_point else np.zeros(zpre.shape, dtype=bool)
    tie = _near_half(x) | zero_tie[:, :, None]
    return GroupQuant(step, zero, q.reshape(rows, k).astype(np.uint8),
                      tie.reshape(rows, k), zero_tie)


def scaled_weights(W: np.ndarray, s_row: np.ndarray) -> np.ndarray:
    """W * diag(s) in binary32 (fp16 weights are exact in binary32).

    [P1] search_scale listing: weight columns are multiplied by s before
    quantizing; [P4] scaling identity: column j of W is multiplied by s_j."""
    return (np.asarray(W, dtype=F16).astype(F32) * np.asarray(s_row, dtype=F32)[None, :]).astype(F32)


# --------------------------------------------------------------------------
# step 4: dequantize and divide by s
# --------------------------------------------------------------------------
def dequantize(gq: GroupQuant, inv_s_row: np.ndarray, group: int = GROUP,
               literal_div: Optional[np.ndarray] = None) -> np.ndarray:
    """fp16 weight of the quantized, unscaled layer.

    [P1] search_scale listing: the quantized scaled weight is divided by s
    ("fold s back"); [P2] "Technical Architecture": Q(W s) s^-1.

    t = binary32((q - zero) * step); the result is t times the binary32
    reciprocal of s, rounded once to fp16 (the product of two binary32 values
    is exact in binary64).  ``literal_div`` (the s row) divides by s instead,
    to measure what the reciprocal changes.
    """
    rows, k = gq.q.shape
    ng = k // group
    step = np.repeat(gq.step, group, axis=1)
    zero = np.repeat(gq.zero, group, axis=1)
    t = ((gq.q.astype(F32) - zero) * step).astype(F32)
    if literal_div is not None:
        return (t.astype(F64) / np.asarray(literal_div, F32).astype(F64)[None, :]).astype(F16)
    prod = t.astype(F64) * np.asarray(inv_s_row, dtype=F32).astype(F64)[None, :]
    return prod.astype(F16)


def fake_quant(W: np.ndarray, s_row: np.ndarray, inv_s_row: np.ndarray,
               group: int = GROUP, w_bit: int = W_BIT, zero_point: bool = True) -> np.ndarray:
    """Q(W diag(s)) diag(s)^-1 as fp16 (steps 3 and 4 together)."""
    return dequantize(quantize(scaled_weights(W, s_row), group, w_bit, zero_point), inv_s_row,
                      group)


# --------------------------------------------------------------------------
# step 5: output error, argmin over the grid
# --------------------------------------------------------------------------
def output_mse(X: np.ndarray, W: np.ndarray, Wq: np.ndarray) -> float:
    """mean over tokens and outputs of (X Wq^T - X W^T)^2, in binary64.

    [P1] search_scale listing: the error is the mean of the squared difference
    between the quantized layer's output and the fp16 layer's output.  The
    reference output is not rounded (fp16 inputs, exact binary64 products).
    """
    X64 = np.asarray(X, F16).astype(F64)
    y_ref = X64 @ np.asarray(W, F16).astype(F64).T
    y = X64 @ np.asarray(Wq, F16).astype(F64).T
    d = y - y_ref
    return float(np.mean(d * d))


def argmin_first(losses: np.ndarray) -> int:
    """Lowest grid index attaining the minimum finite loss.

    [P1] search_scale listing: the best error starts at +inf and is replaced
    only on a strictly smaller error, so the first minimum wins and a NaN
    never wins.  No finite loss means no scale is chosen (raised here).
    """
    best, best_i = np.inf, -1
    for i, v in enumerate(np.asarray(losses, dtype=F64)):
        if v < best:
            best, best_i = v, i
    if best_i < 0:
        raise NonFiniteLosses("no finite loss on the grid")
    return best_i


@dataclass
class SearchResult:
    losses: np.ndarray      # [n_grid] float64
    best: int               # argmin index
    s_best: np.ndarray      # [in] float32
    s: np.ndarray           # [n_grid, in] float32
    inv_s: np.ndarray       # [n_grid, in] float32


def search_layer(X: np.ndarray, W: np.ndarray, sal: np.ndarray, n_grid: int = N_GRID,
                 floor: float = SAL_FLOOR, group: int = GROUP, w_bit: int = W_BIT,
                 zero_point: bool = True, row_chunk: Optional[int] = None) -> SearchResult:
    """The per-layer grid search, in the order of [P1]'s search_scale listing:
    reference output; for each alpha: scale, quantize, fold back, output MSE;
    keep the first strict minimum.

    ``row_chunk`` runs the same steps on blocks of that many output rows at a
    time and adds each block's sum of squared differences (the quantizer
    works row by row, so a block's codes are those of the whole layer); the
    loss is the total over all N * out outputs divided by their count.  It
    only bounds the memory the large layers need; without it the layer is one
    block."""
    s, inv_s = scale_table(sal, n_grid, floor)
    X64 = np.asarray(X, F16).astype(F64)
    W = np.asarray(W, F16)
    n_out = W.shape[0]
    chunk = n_out if row_chunk is None else int(row_chunk)
    if chunk <= 0:
        raise ValueError("row_chunk must be positive")
    sums = np.zeros(n_grid, dtype=F64)
    for o0 in range(0, n_out, chunk):
        Wc = W[o0:o0 + chunk]
        y_ref = X64 @ Wc.astype(F64).T
        for i in range(n_grid):
            wq = fake_quant(Wc, s[i], inv_s[i], group, w_bit, zero_point)
            d = X64 @ wq.astype(F64).T - y_ref
            sums[i] += np.sum(d * d)
    losses = sums / F64(X64.shape[0] * n_out)
    best = argmin_first(losses)
    return SearchResult(losses, best, s[best].copy(), s, inv_s)


def tile_sq_error(X: np.ndarray, W: np.ndarray, s_row: np.ndarray, inv_s_row: np.ndarray,
                  rows: slice, cols: slice, group: int = GROUP, w_bit: int = W_BIT,
                  zero_point: bool = True) -> float:
    """Sum of squared output differences over a token range x output range.

    The same quantity as output_mse restricted to a sub-block (not divided by
    its size): a large layer's loss is the sum of such blocks, which lets a
    test check a large run one block at a time.
    """
    Wsub = np.asarray(W, F16)[cols]
    wq = fake_quant(Wsub, s_row, inv_s_row, group, w_bit, zero_point)
    X64 = np.asarray(X, F16)[rows].astype(F64)
    d = X64 @ wq.astype(F64).T - X64 @ Wsub.astype(F64).T
    return float(np.sum(d * d))


# --------------------------------------------------------------------------
# packing the chosen codes
# --------------------------------------------------------------------------
@dataclass
class Packed:
    qweight: np.ndarray   # [out, in/8] int32, nibble j of word w = code of column 8w+j
    step16: np.ndarray    # [out, in/group] float16
    zero16: np.ndarray    # [out, in/group] float16
    q: np.ndarray         # [out, in] uint8 (unpacked codes)
    tie: np.ndarray       # [out, in] bool (see GroupQuant.tie)
    zero_tie: np.ndarray  # [out, in/group] bool (see GroupQuant.zero_tie)


def pack_codes(q: np.ndarray) -> np.ndarray:
    """Eight 4-bit codes per 32-bit word along in_features, lowest column in
    the lowest nibble ([P2] pipeline step "INT4 Weight Packing & Export":
    INT4 codes live in INT32 containers; the nibble order is our reading)."""
    q = np.asarray(q, dtype=np.uint32)
    rows, k = q.shape
    q = q.reshape(rows, k // 8, 8)
    word = np.zeros((rows, k // 8), dtype=np.uint32)
    for j in range(8):
        word |= (q[:, :, j] & np.uint32(0xF)) << np.uint32(4 * j)
    return word.view(np.int32)


def unpack_codes(qweight: np.ndarray) -> np.ndarray:
    w = np.asarray(qweight).view(np.uint32)
    rows, kw = w.shape
    out = np.empty((rows, kw, 8), dtype=np.uint8)
    for j in range(8):
        out[:, :, j] = (w >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(rows, kw * 8)


def pack(W: np.ndarray, s_row: np.ndarray, group: int = GROUP, w_bit: int = W_BIT,
         zero_point: bool = True) -> Packed:
    """Quantize W diag(s) with exact division and pack the codes, with the
    per-group step and zero point stored as fp16 ([P1] quant_config;
    [P3] worked example: one 16-bit scale per 128 weights).  Codes of fewer
    than 4 bits still take one nibble each."""
    gq = quantize(scaled_weights(W, s_row), group, w_bit, zero_point)
    return Packed(pack_codes(gq.q), gq.step.astype(F16), gq.zero.astype(F16), gq.q, gq.tie,
                  gq.zero_tie)


def packed_bytes(n_weights: int, group: int = GROUP, w_bit: int = W_BIT) -> dict:
    """Storage of the packed format for n_weights weights (codes, steps, zeros)."""
    return {
        "codes": n_weights * w_bit // 8,
        "steps": n_weights // group * 2,
        "zeros": n_weights // group * 2,
        "fp16": n_weights * 2,
    }


# --------------------------------------------------------------------------
# inference with the packed weights: W4A16 product y = x Wdq^T
# --------------------------------------------------------------------------
def dequant_packed(qweight: np.ndarray, step16: np.ndarray, zero16: np.ndarray,
                   group: int = GROUP) -> np.ndarray:
    """The real-valued weight the packed format stands for, (q - z) * step per
    element, exact in binary64 (q a 4-bit code, z and step the stored fp16
    values of the element's group): the inverse map of the step-size
    equation of [P4], applied to the INT32-packed codes of [P2]."""
    q = unpack_codes(qweight).astype(F64)
    st = np.repeat(np.asarray(step16, F16).astype(F64), group, axis=1)
    zr = np.repeat(np.asarray(zero16, F16).astype(F64), group, axis=1)
    return (q - zr) * st


def w4a16_matmul(x: np.ndarray, qweight: np.ndarray, step16: np.ndarray, zero16: np.ndarray,
                 group: int = GROUP) -> np.ndarray:
    """Decode-time product of fp16 activations with the packed 4-bit weights
    (W4A16, [P1] "What do you actually deploy": 4-bit weights, 16-bit
    activations, groups of 128 with a zero point; decode streams the packed
    weights instead of fp16 ones): y[t, o] = sum_k x[t, k] (q[o, k] - z) step,
    in binary64.  The activations are whatever the caller feeds the layer
    (after the 1/s fold, x / s)."""
    return np.asarray(x, F16).astype(F64) @ dequant_packed(qweight, step16, zero16, group).T


def w4a16_abs_matmul(x: np.ndarray, qweight: np.ndarray, step16: np.ndarray,
                     zero16: np.ndarray, group: int = GROUP) -> np.ndarray:
    """sum_k |x[t, k]| (|q| + |z|) |step|: the scale of the rounding-error
    bound of any binary32 evaluation of w4a16_matmul (error bounds only)."""
    q = unpack_codes(qweight).astype(F64)
    st = np.abs(np.repeat(np.asarray(step16, F16).astype(F64), group, axis=1))
    zr = np.abs(np.repeat(np.asarray(zero16, F16).astype(F64), group, axis=1))
    return np.abs(np.asarray(x, F16).astype(F64)) @ ((q + zr) * st).T


# --------------------------------------------------------------------------
# folding 1/s into the operation that feeds the layer
# --------------------------------------------------------------------------
def fold_inverse_scale(src16: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Row j of src divided by s_j: dst = fp16(fp32(src) / s) row-wise.

    The inverse of the per-channel scale is absorbed by whatever produces the
    layer's input channels ([P4] "Salient Weight Preservation": the preceding
    normalization's per-channel scale times 1/s_j; [P5] "Per-channel scaling":
    the inverse is fused into preceding layers).  Rows are the layer's input
    channels: a norm's gain or bias is a [n] (or [n, 1]) array, a preceding
    linear's weight is [n, cols] and its bias [n].  The quotient is a binary32
    division, rounded to fp16 (overflow gives an infinity)."""
    a = np.asarray(src16, F16)
    s = np.asarray(s, F32)
    col = s.reshape((-1,) + (1,) * (a.ndim - 1))
    with np.errstate(over="ignore"):
        return (a.astype(F32) / col).astype(F32).astype(F16)


# --------------------------------------------------------------------------
# saliency ablations
# --------------------------------------------------------------------------
def weight_saliency(W: np.ndarray) -> np.ndarray:
    """Saliency from weight magnitude instead of activations: the mean of
    |W[o, k]| over output rows ([P1] "How does AWQ decide which weights to
    protect?" contrasts this choice with activation magnitude).  The same
    exact column mean as act_stats, taken over W's rows."""
    return act_stats(np.asarray(W, F16))


def select_top_channels(sal: np.ndarray, n_keep: int) -> np.ndarray:
    """Keep the saliency of the n_keep most salient channels and set the rest
    to 1, so that only those channels are scaled (s = 1^alpha = 1 elsewhere):
    the "top ~1% of channels" reading of [P1] (protecting about 1% recovers
    most of the accuracy) and [P2] (the top 1% weight channels are scaled).
    Larger saliency first; equal values go to the lower channel index."""
    sal = np.asarray(sal, F32)
    n = sal.shape[0]
    if not 0 <= n_keep <= n:
        raise ValueError("n_keep outside 0..n")
    order = np.lexsort((np.arange(n), -sal.astype(F64)))
    out = np.ones(n, F32)
    keep = order[:n_keep]
    out[keep] = sal[keep]
    return out
