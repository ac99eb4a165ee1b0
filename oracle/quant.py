"""CPU oracle of the step that produces the grouped matmul's inputs: dynamic
per-token int8 quantisation of bf16 hidden states and the routing permute.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this module.  It shares no code with
the GPU library.

The pages name this step without its formulas: the all-to-all grouped matmul
page ("aclnnAlltoAllvQuantGroupedMatMul", function and formula; quantisation
modes) lists a dispatch-and-permute stage before the expert matmul and a
"pertoken dynamic quantisation" mode; the PTOAS issue (#1568, background) shows
a per-token bf16 cast that multiplies each value by an inverse scale; the
per-token matmul page ("matmul支持pertoken量化模式", inputs) fixes what the
matmul then takes: int8 x with one float perTokenScale per row.  Readings taken
(plain symmetric int8, round to nearest even):

  1. per token t, over its k values x (bf16 widened to fp32, exact):
       amax_t  = max_j |x[t][j]|
       scale_t = fl(amax_t / 127)            (the dequant step: x ~ q * scale)
       inv_t   = fl(127 / amax_t), 0 when amax_t = 0
       q[t][j] = clamp(rne(fl(x[t][j] * inv_t)), -127, 127)
  2. entry f = t*K + j routes token t to global expert ids[t][j]; its local
     expert is g = ids[t][j] - expert_offset; entries with g outside [0, e)
     belong to other ranks and produce no row.
  3. rows are the local entries sorted by g, ties in ascending f (a stable
     sort); row i holding entry f = t*K + j gets
       x1[i] = q[t], pertokenScale[i] = scale_t, logit[i] = weights[t][j],
       rowIndex[i] = t.
  4. groupList[g] = rows of expert g (type 1) or the cumulative end (type 0).

Rows at and past sum(counts) are not defined (the grouped matmul never reads
them).  Hidden values must be finite.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 (the upper half of the binary32 word)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize(hidden_bits):
    """Step 1: (q int8 (T,k), scale float32 (T)) from bf16 bits (T,k)."""
    x = bf16_to_f32(hidden_bits)
    if x.shape[1] == 0:
        return np.zeros(x.shape, dtype=np.int8), np.zeros(x.shape[0], dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    if not np.isfinite(amax).all():
        raise ValueError("hidden values must be finite")
    scale = (amax / np.float32(127.0)).astype(np.float32)
    inv = np.zeros_like(amax)
    nz = amax > 0
    inv[nz] = np.float32(127.0) / amax[nz]
    prod = (x * inv[:, None]).astype(np.float32)
    q = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    return q, scale


def permute(expert_ids, e: int, expert_offset: int = 0):
    """Steps 2-3 on the indices: (order of flat entries f, counts (e))."""
    ids = np.asarray(expert_ids).astype(np.int64).reshape(-1)
    g = ids - int(expert_offset)
    f = np.nonzero((g >= 0) & (g < e))[0]
    order = f[np.argsort(g[f], kind="stable")]
    counts = np.bincount(g[f], minlength=e).astype(np.int64)
    return order, counts


def run(rp):
    """All four steps.  Returns a dict: x1 (m,k) int8, pertoken_scale (m),
    logit (m) or None, row_index (m) int64, group_list (e) int64, and
    ``rows`` = sum(counts); entries at and past ``rows`` are zero here and
    undefined in the operator."""
    T, K, k, e = int(rp.T), int(rp.K), int(rp.k), int(rp.e)
    if np.asarray(rp.hidden).shape != (T, k) or np.asarray(rp.expert_ids).shape != (T, K):
        raise ValueError("shapes")
    if rp.group_list_type not in (0, 1):
        raise ValueError("groupListType")
    q, scale = quantize(rp.hidden)
    order, counts = permute(rp.expert_ids, e, rp.expert_offset)
    m = T * K
    rows = len(order)
    tok = order // K if K > 0 else order
    x1 = np.zeros((m, k), dtype=np.int8)
    x1[:rows] = q[tok]
    pts = np.zeros(m, dtype=np.float32)
    pts[:rows] = scale[tok]
    ri = np.zeros(m, dtype=np.int64)
    ri[:rows] = tok
    logit = None
    if rp.topk_weights is not None:
        logit = np.zeros(m, dtype=np.float32)
        logit[:rows] = np.asarray(rp.topk_weights, dtype=np.float32).reshape(-1)[order]
    gl = np.cumsum(counts).astype(np.int64) if rp.group_list_type == 0 else counts.copy()
    return dict(x1=x1, pertoken_scale=pts, logit=logit, row_index=ri, group_list=gl, rows=rows,
                scale_per_token=scale, q_per_token=q)
