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

FP8 outputs (for the FP8 and MxA8W4 grouped matmuls; readings, the pages
giving only the mode names and the multiply by an inverse scale):
  fp8 per token:  scale_t = fl(amax_t / 448), inv = fl(448 / amax_t) (0 when
                  amax_t = 0), code = E4M3(fl(x * inv)), 448 being the
                  largest finite E4M3 value;
  mx (per 32 k):  the OCP MX v1.0 conversion: for each block of 32 values of a
                  token, shared exponent s = floor(log2(amax_b)) - 8 (8 = the
                  largest E4M3 exponent), clamped to [-127, 127] (-127 for an
                  all-zero block), E8M0 code s + 127, element code
                  E4M3(clamp(x * 2^-s, -448, 448)).
E4M3(v) rounds to the nearest E4M3 value, ties to the even code.
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


_E4M3_CODES = np.arange(0x00, 0x7F)  # non-negative finite codes (0x7F is NaN)


def _e4m3_values():
    from .mx import FP8_TABLE  # decoded from the format definition
    return FP8_TABLE[_E4M3_CODES]


def e4m3_encode(v):
    """FP8 E4M3 codes (uint8) of finite values with |v| <= 448: nearest
    representable value, ties to the even code; the sign bit from v."""
    vals = _e4m3_values()
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if (a > 448.0).any():
        raise ValueError("E4M3 encode: value beyond 448")
    hi = np.clip(np.searchsorted(vals, a, side="left"), 1, len(vals) - 1)
    lo = hi - 1
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(_E4M3_CODES[lo] % 2 == 0, lo, hi)))
    code = _E4M3_CODES[pick].astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 7)


def quantize_fp8(hidden_bits):
    """FP8 per token: (codes uint8 (T,k), scale float32 (T))."""
    x = bf16_to_f32(hidden_bits)
    amax = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    if not np.isfinite(amax).all():
        raise ValueError("hidden values must be finite")
    scale = (amax / np.float32(448.0)).astype(np.float32)
    inv = np.zeros_like(amax)
    nz = amax > 0
    inv[nz] = np.float32(448.0) / amax[nz]
    prod = (x * inv[:, None]).astype(np.float32)
    return e4m3_encode(np.clip(prod, -448.0, 448.0)), scale


def quantize_mx(hidden_bits):
    """MX per 32 values: (codes uint8 (T,k), E8M0 codes uint8 (T, k/32))."""
    x = bf16_to_f32(hidden_bits).astype(np.float64)
    T, k = x.shape
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    xb = x.reshape(T, k // 32, 32)
    amax = np.abs(xb).max(axis=2)
    if not np.isfinite(amax).all():
        raise ValueError("hidden values must be finite")
    _, ex = np.frexp(amax)                      # amax = f * 2^ex, f in [0.5, 1)
    s = np.where(amax > 0, ex - 1 - 8, -127)    # floor(log2(amax)) - 8
    s = np.clip(s, -127, 127)
    v = np.clip(xb * np.exp2(-s)[:, :, None], -448.0, 448.0)  # exact: a power-of-two scaling
    return e4m3_encode(v).reshape(T, k), (s + 127).astype(np.uint8)


def permute(expert_ids, e: int, expert_offset: int = 0):
    """Steps 2-3 on the indices: (order of flat entries f, counts (e))."""
    ids = np.asarray(expert_ids).astype(np.int64).reshape(-1)
    g = ids - int(expert_offset)
    f = np.nonzero((g >= 0) & (g < e))[0]
    order = f[np.argsort(g[f], kind="stable")]
    counts = np.bincount(g[f], minlength=e).astype(np.int64)
    return order, counts


def run(rp):
    """All four steps.  Returns a dict: x1 (m,k) int8 (FP8 modes: uint8 E4M3
    codes), pertoken_scale (m) float32 (mx: uint8 E8M0 codes (m, k/32)),
    logit (m) or None, row_index (m) int64, group_list (e) int64, and
    ``rows`` = sum(counts); entries at and past ``rows`` are zero here and
    undefined in the operator."""
    T, K, k, e = int(rp.T), int(rp.K), int(rp.k), int(rp.e)
    if np.asarray(rp.hidden).shape != (T, k) or np.asarray(rp.expert_ids).shape != (T, K):
        raise ValueError("shapes")
    if rp.group_list_type not in (0, 1):
        raise ValueError("groupListType")
    mode = getattr(rp, "mode", "int8")
    if mode == "int8":
        q, scale = quantize(rp.hidden)
    elif mode == "fp8":
        q, scale = quantize_fp8(rp.hidden)
    elif mode == "mx":
        q, scale = quantize_mx(rp.hidden)
    else:
        raise ValueError(mode)
    order, counts = permute(rp.expert_ids, e, rp.expert_offset)
    m = T * K
    rows = len(order)
    tok = order // K if K > 0 else order
    x1 = np.zeros((m, k), dtype=q.dtype)
    x1[:rows] = q[tok]
    pts = np.zeros((m,) + scale.shape[1:], dtype=scale.dtype)
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
