"""CPU oracle for the MxA8W4 and FP8 modes.  TEST INFRASTRUCTURE ONLY: the tests, the
smoke check and the CPU-baseline leg of the benchmark may use it; the GPU
library never does, and the two share no code.

What it computes ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2", Atlas 350
notes on the MxA8W4 quantisation: x2 given as (e,n,k) with transposeX2 fixed
true, pertokenScale of shape (m, ceil(k/64), 2) required, scale of shape
(e, n, ceil(k/64), 2); the page's dtype table is lost, and the reading taken is
x1 FLOAT8_E4M3FN, x2 FLOAT4_E2M1 two per byte along k, both scales
FLOAT8_E8M0, one scale per 32 consecutive k; the page asks k % 32 == 0, so
when k % 64 == 32 the second byte of each row's last scale pair stands for no
block and is not read):

    acc[i][j] = sum_kk x1[i][kk] * 2^(pts[i][kk//32] - 127) * w[g][j][kk] * 2^(scale[g][j][kk//32] - 127)
    y[i][j]   = acc[i][j] * logit[i]
    out[d]    = seed[d] + sum of y[i] over covered rows i with rowIndex[i] = d (ascending i)

for row i of expert g, groups and the seed as in the int8 mode.  Everything is
evaluated in float64: each scaled product is exact there (at most 6
significant bits, exponents within range), and a matrix product of such terms
is a library step.  The GPU's matrix core does not round like fp32 inside an
instruction, so parity is judged against an error bound (``bound``) derived
from its arithmetic, measured on the device with constructed inputs: within
one 32-k scale block the products are aligned to the largest one and kept to
about 13 bits below it (a product 2^-14 below the largest of its block is
dropped, one 2^-13 below is kept), the block sums are added into the fp32
accumulator with round-to-nearest-even.  Taken with one bit of margin, a block
contributes at most 32 * 2^(e - 12) <= 2^-7 * max|product| of error (e the
exponent of its largest product), bounded above by 2^-7 * max|x1 block| *
max|w block|; the k/32 block sums and the accumulator then add like fp32.

FP8 mode (x1 and x2 FLOAT8_E4M3FN, "aclnnGroupedMatmulFinalizeRoutingWeightNzV2"
parameter notes: rowIndex INT64 only for FLOAT8_E4M3FN inputs; Atlas 350
pertoken-perchannel quantisation): x2 given as (e,n,k) here, no block scales,
and the int8 mode's dequantisation after the sum:

    acc[i][j] = sum_kk x1[i][kk] * w[g][j][kk]
    y[i][j]   = ((acc[i][j] * scale[g][0][j]) * pertokenScale[i]) * logit[i]

Element formats (OCP Microscaling formats, v1.0, element data types):
    FP8 E4M3: sign, 4-bit exponent (bias 7), 3-bit mantissa; exponent 0 is
              subnormal (2^-6 * m/8); exponent 15 with mantissa 7 is NaN.
    FP4 E2M1: sign, 2-bit exponent (bias 1), 1-bit mantissa; exponent 0 is
              subnormal (m/2).
    E8M0:     2^(b - 127); b = 255 is NaN.
"""
from __future__ import annotations

import math

import numpy as np

U32 = 2.0 ** -23  # fp32 unit roundoff, taken at its directed-rounding size


def fp8_e4m3_value(code: int) -> float:
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    mag = math.ldexp(1.0 + m / 8.0, e - 7) if e else math.ldexp(m / 8.0, -6)
    return -mag if s else mag


def fp4_e2m1_value(code: int) -> float:
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = math.ldexp(1.0 + m / 2.0, e - 1) if e else m / 2.0
    return -mag if s else mag


def e8m0_value(b: int) -> float:
    return math.nan if b == 255 else math.ldexp(1.0, b - 127)


FP8_TABLE = np.array([fp8_e4m3_value(c) for c in range(256)], dtype=np.float64)
FP4_TABLE = np.array([fp4_e2m1_value(c) for c in range(16)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)


def unpack_fp4(pairs: np.ndarray) -> np.ndarray:
    """(..., k/2) bytes -> (..., k) codes; the low nibble is the even k."""
    pairs = np.asarray(pairs, dtype=np.uint8)
    out = np.empty(pairs.shape[:-1] + (pairs.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = pairs & 0xF
    out[..., 1::2] = pairs >> 4
    return out


def group_ranges(p):
    """[start_g, end_g) of every expert (groupList type 0: cumulative ends,
    type 1: counts).  Raises on a list that breaks its rule or exceeds m."""
    gl = np.asarray(p.group_list, dtype=np.int64)
    if p.group_list_type == 0:
        ends = gl
        if (ends < 0).any() or (np.diff(ends) < 0).any():
            raise ValueError("groupList (cumulative) must be non-negative and non-decreasing")
    else:
        if (gl < 0).any():
            raise ValueError("groupList (counts) must be non-negative")
        ends = np.cumsum(gl)
    if ends.size and ends[-1] > p.m:
        raise ValueError("groupList covers more than m rows")
    starts = np.concatenate([[0], ends[:-1]]).astype(np.int64)
    return starts, ends.astype(np.int64)


def _is_fp8(p) -> bool:
    return bool(getattr(p, "fp8", False))


def _scaled_rows(p, rows):
    """x1 rows with their block scales applied (MX) or as decoded (FP8), float64 (len(rows), k)."""
    x = FP8_TABLE[np.asarray(p.x1)[rows]]
    if _is_fp8(p):
        return x
    # (rows, ceil(k/64)*2) bytes; the first k/32 are the blocks' scales (when
    # k % 64 == 32 the last pair's second byte stands for no block)
    s = E8M0_TABLE[np.asarray(p.pertoken_scale)[rows]].reshape(len(rows), -1)[:, :p.k // 32]
    return x * np.repeat(s, 32, axis=1)


def _scaled_weights(p, g):
    """Expert g's weights with their block scales applied (MX) or as decoded (FP8), float64 (n, k)."""
    if _is_fp8(p):
        # (e,n,k) when given transposed, else (e,k,n) ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2",
        # full-quant notes: x2 may be transposed or not)
        w = np.asarray(p.x2)[g]
        return FP8_TABLE[w if getattr(p, "x2_transposed", True) else w.T]
    w = FP4_TABLE[unpack_fp4(np.asarray(p.x2)[g])]
    s = E8M0_TABLE[np.asarray(p.scale)[g]].reshape(p.n, -1)[:, :p.k // 32]  # (n, k/32), as for the rows
    return w * np.repeat(s, 32, axis=1)


def _gamma(t: int) -> float:
    return t * U32 / (1.0 - t * U32)


def rows_acc(p, rows, g):
    """acc (float64), the sum of |terms| and the sum over 32-k blocks of
    max|x1 block| * max|w block| (an upper bound of the blocks' largest
    products) for the listed rows of expert g."""
    a = _scaled_rows(p, rows)
    w = _scaled_weights(p, g)
    amax = np.abs(a).reshape(a.shape[0], -1, 32).max(axis=2)
    wmax = np.abs(w).reshape(w.shape[0], -1, 32).max(axis=2)
    return a @ w.T, (np.abs(a) @ np.abs(w).T, amax @ wmax.T)


def _post(p, rows, g):
    """The factors applied after the sum, as one float64 multiplier per element,
    and the number of rounded fp32 products that apply them: MX logit only;
    FP8 ((acc * scale) * pertokenScale) * logit."""
    rows = np.asarray(rows)
    L = np.ones(len(rows)) if p.logit is None else np.asarray(p.logit, dtype=np.float64)[rows]
    if not _is_fp8(p):
        return np.repeat(L[:, None], p.n, axis=1), 1
    if p.pertoken_scale is None:
        P = np.ones(len(rows))
    else:  # per token, or one static per-tensor value for every row
        pts = np.asarray(p.pertoken_scale, dtype=np.float64)
        P = pts[rows] if len(pts) > 1 else np.full(len(rows), pts[0])
    if p.scale is None:
        S = np.ones(p.n)
    elif p.scale_bf16:
        S = (np.asarray(p.scale)[g, 0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        S = np.asarray(p.scale, dtype=np.float64)[g, 0]
    return S[None, :] * P[:, None] * L[:, None], 3


def _seed_row(p, d):
    row = np.zeros(p.n, dtype=np.float64)
    if p.shared_input is not None and p.shared_input_offset <= d < p.shared_input_offset + p.bsdp:
        bits = np.asarray(p.shared_input)[d - p.shared_input_offset].astype(np.uint32) << 16
        row = bits.view(np.float32).astype(np.float64)
    return row


def run(p):
    """Whole computation.  Returns (out, bound, acc): out and acc in float64,
    bound the per-element limit of |gpu - out| for an fp32 evaluation in any
    order (see ``_row_error`` and the fold below)."""
    starts, ends = group_ranges(p)
    acc = np.zeros((p.m, p.n), dtype=np.float64)
    mag = np.zeros((p.m, p.n), dtype=np.float64)
    bmax = np.zeros((p.m, p.n), dtype=np.float64)
    for g in range(p.e):
        if ends[g] > starts[g]:
            rows = np.arange(starts[g], ends[g])
            acc[rows], (mag[rows], bmax[rows]) = rows_acc(p, rows, g)
    covered = np.zeros(p.m, dtype=bool)
    for a, b in zip(starts, ends):
        covered[a:b] = True
    y = np.zeros_like(acc)
    ey = np.zeros_like(acc)
    for g in range(p.e):
        if ends[g] > starts[g]:
            rows = np.arange(starts[g], ends[g])
            mult, nmul = _post(p, rows, g)
            y[rows] = acc[rows] * mult
            ey[rows] = _row_error(acc[rows], mag[rows], bmax[rows], mult, nmul, p.k)
    ri = np.arange(p.m) if p.row_index is None else np.asarray(p.row_index, dtype=np.int64)
    out = np.stack([_seed_row(p, d) for d in range(p.output_bs)]) if p.output_bs else np.zeros((0, p.n))
    err = np.zeros_like(out)
    absum = np.abs(out)
    terms = np.zeros(p.output_bs, dtype=np.int64)
    for i in range(p.m):  # ascending source order
        if not covered[i]:
            continue
        d = ri[i]
        if not 0 <= d < p.output_bs:
            raise ValueError("rowIndex outside [0, outputBS)")
        out[d] += y[i]
        err[d] += ey[i]
        absum[d] += np.abs(y[i]) + ey[i]
        terms[d] += 1
    bound = err + np.array([_gamma(int(t)) for t in terms])[:, None] * absum
    return out, bound, acc


def _row_error(acc, mag, bmax, mult, nmul, k):
    """|y_gpu - acc*mult| <= |mult| (E + gamma_nmul (|acc| + E)) with
    E = 2^-7 bmax + gamma_(k/32+1) (mag + 2^-7 bmax): the in-block alignment
    of the matrix core, the fp32 additions of the block sums, then nmul
    rounded products."""
    e_blk = 2.0 ** -7 * bmax
    e_acc = e_blk + _gamma(k // 32 + 1) * (mag + e_blk)
    return np.abs(mult) * (e_acc + _gamma(nmul) * (np.abs(acc) + e_acc))


def out_rows(p, d_list):
    """(out, bound) for the listed destination rows only (full-size checks).
    The contributing rows are evaluated expert by expert (one weight decode per
    expert), then folded per destination in ascending row order."""
    starts, ends = group_ranges(p)
    group_of = np.full(p.m, -1, dtype=np.int64)
    for g in range(p.e):
        group_of[starts[g]:ends[g]] = g
    ri = np.arange(p.m) if p.row_index is None else np.asarray(p.row_index, dtype=np.int64)
    d_list = [int(d) for d in d_list]
    rows_of = {d: np.nonzero((ri == d) & (group_of >= 0))[0] for d in d_list}  # ascending
    need = np.unique(np.concatenate([rows_of[d] for d in d_list] + [np.zeros(0, dtype=np.int64)]))
    y, ey = {}, {}
    for g in np.unique(group_of[need]):
        rows = need[group_of[need] == g]
        a, (m_, b_) = rows_acc(p, rows, int(g))
        mult, nmul = _post(p, rows, int(g))
        yr = a * mult
        er = _row_error(a, m_, b_, mult, nmul, p.k)
        for t, i in enumerate(rows):
            y[int(i)], ey[int(i)] = yr[t], er[t]
    outs, bounds = [], []
    for d in d_list:
        o = _seed_row(p, d)
        err = np.zeros(p.n)
        absum = np.abs(o)
        for i in rows_of[d]:
            o = o + y[int(i)]
            err += ey[int(i)]
            absum += np.abs(y[int(i)]) + ey[int(i)]
        outs.append(o)
        bounds.append(err + _gamma(len(rows_of[d])) * absum)
    return np.array(outs), np.array(bounds)


def brute(p):
    """Pure-Python evaluation of acc from the element definitions, for tiny
    problems (an independent reading of the decoding and the block scales)."""
    starts, ends = group_ranges(p)
    x1 = np.asarray(p.x1)
    x2 = np.asarray(p.x2)
    sa = np.asarray(p.pertoken_scale)
    sb = np.asarray(p.scale)
    acc = [[0.0] * p.n for _ in range(p.m)]
    for g in range(p.e):
        for i in range(int(starts[g]), int(ends[g])):
            for j in range(p.n):
                total = 0.0
                for kk in range(p.k):
                    if _is_fp8(p):  # both operands FP8, no block scales; x2 (e,n,k) or (e,k,n)
                        wb = x2[g, j, kk] if getattr(p, "x2_transposed", True) else x2[g, kk, j]
                        total += fp8_e4m3_value(int(x1[i, kk])) * fp8_e4m3_value(int(wb))
                        continue
                    byte = int(x2[g, j, kk // 2])
                    wcode = byte & 0xF if kk % 2 == 0 else byte >> 4
                    blk = kk // 32
                    a = fp8_e4m3_value(int(x1[i, kk])) * e8m0_value(int(sa[i, blk // 2, blk % 2]))
                    b = fp4_e2m1_value(wcode) * e8m0_value(int(sb[g, j, blk // 2, blk % 2]))
                    total += a * b
                acc[i][j] = total
    return np.array(acc, dtype=np.float64)
