"""Pure-Python brute force of the same definition, for tiny inputs.

TEST INFRASTRUCTURE ONLY.  Written separately from the C oracle so that an
indexing or decoding mistake in either one shows up as a disagreement.
Integers are Python ints (exact); every float step is one numpy.float32
operation (IEEE binary32, round to nearest even), in the order
((float(acc) * scale) * pertokenScale) * logit, and the combine adds the
covered source rows of each destination in ascending row order onto the seed.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def _bf16(bits: int) -> np.float32:
    return np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0]


def _weight(p, g: int, kk: int, j: int) -> int:
    if getattr(p, "x2_transposed", False):  # int8 (e,n,k): column j holds k contiguous values
        return int(p.x2[g, j, kk])
    if not p.x2_int4:
        return int(p.x2[g, kk, j])
    word = int(p.x2[g, kk, j // 8]) & 0xFFFFFFFF
    nib = (word >> (4 * (j % 8))) & 0xF
    return nib - 16 if nib >= 8 else nib


def _scale(p, g: int, j: int) -> np.float32:
    if p.scale is None:
        return F32(1.0)
    v = p.scale[g, 0, j]
    return _bf16(v) if p.scale_bf16 else F32(v)


def ranges(p):
    """Group ranges per the groupList rule (type 0 cumulative, type 1 counts)."""
    out = []
    prev = 0
    for g in range(p.e):
        v = int(p.group_list[g])
        if v < 0:
            raise ValueError("negative groupList entry")
        if p.group_list_type == 0:
            if v < prev:
                raise ValueError("cumulative groupList decreases")
            s, e = prev, v
        elif p.group_list_type == 1:
            s, e = prev, prev + v
        else:
            raise ValueError("groupListType must be 0 or 1")
        if e > p.m:
            raise ValueError("groupList covers more rows than x1 has")
        out.append((s, e))
        prev = e
    return out


def brute(p):
    """Returns (out as float32 (outputBS,n), acc as int64 (m,n))."""
    m, k, n = p.m, p.k, p.n
    acc = np.zeros((m, n), dtype=np.int64)
    group = [-1] * m
    for g, (s, e) in enumerate(ranges(p)):
        for i in range(s, e):
            group[i] = g
    for i in range(m):
        g = group[i]
        if g < 0:
            continue
        for j in range(n):
            acc[i, j] = sum(int(p.x1[i, kk]) * _weight(p, g, kk, j) for kk in range(k))
    out = np.zeros((p.output_bs, n), dtype=np.float32)
    if p.shared_input is not None:
        off = int(p.shared_input_offset)
        for r in range(p.shared_input.shape[0]):
            for j in range(n):
                out[off + r, j] = _bf16(p.shared_input[r, j])
    for i in range(m):
        g = group[i]
        if g < 0:
            continue
        d = i if p.row_index is None else int(p.row_index[i])
        if not 0 <= d < p.output_bs:
            raise ValueError("rowIndex outside the output")
        # per token, or one static per-tensor value for every row
        P = F32(1.0) if p.pertoken_scale is None else F32(p.pertoken_scale[i if len(p.pertoken_scale) > 1 else 0])
        L = F32(1.0) if p.logit is None else F32(p.logit[i])
        for j in range(n):
            y = F32(int(acc[i, j]))
            y = F32(y * _scale(p, g, j))
            y = F32(y * P)
            y = F32(y * L)
            out[d, j] = F32(out[d, j] + y)
    return out, acc
