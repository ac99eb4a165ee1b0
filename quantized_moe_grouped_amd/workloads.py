"""Seeded synthetic inputs for the grouped quantized MoE matmul + finalize-routing.

This module only draws and encodes inputs (numpy, host memory).  It holds none
of the method's arithmetic: no matmul, no dequantisation, no combine.  Both the
GPU path's tests and the CPU oracle's tests take their inputs from here.

Layouts follow the operator's parameter description
("aclnnGroupedMatmulFinalizeRoutingWeightNzV2", parameter notes for Atlas
A2/A3 and the Atlas 350 common constraints):
  x1 int8 (m,k); x2 int8 (e,k,n) or int4 packed eight per int32 (e,k,n/8);
  scale fp32 or bf16 (e,1,n); pertokenScale fp32 (m); logit fp32 (m);
  groupList int64 (e) of type 0 (cumulative) or 1 (counts); rowIndex int64 or
  int32 (m); sharedInput bf16 (bsdp,n) placed at sharedInputOffset inside an
  output of outputBS rows.

bf16 arrays are carried as their raw uint16 bit patterns.

Every draw uses ``numpy.random.default_rng(seed)`` in a fixed order:
counts -> rowIndex -> logit -> x1 -> x2 -> scale -> pertokenScale -> sharedInput.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# ---------------------------------------------------------------- encodings


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> fp32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def pack_int4(values: np.ndarray) -> np.ndarray:
    """Pack signed int4 values (..., n) in [-8, 7] into int32 words (..., n/8).

    Column 8w+t goes to bits [4t, 4t+4) of word w (low nibble first), two's
    complement -- the (e,k,n) <-> (e,k,n/8) correspondence of the operator's
    parameter notes, with the nibble order read as little-endian.
    """
    v = np.asarray(values)
    if v.shape[-1] % 8:
        raise ValueError("last dimension must be a multiple of 8")
    if v.min(initial=0) < -8 or v.max(initial=0) > 7:
        raise ValueError("int4 values must lie in [-8, 7]")
    nib = (v.astype(np.int64) & 0xF).astype(np.uint64)
    nib = nib.reshape(*v.shape[:-1], v.shape[-1] // 8, 8)
    shifts = (np.arange(8, dtype=np.uint64) * 4)
    words = (nib << shifts).sum(axis=-1, dtype=np.uint64).astype(np.uint32)
    return words.view(np.int32)


# ---------------------------------------------------------------- container


@dataclasses.dataclass
class Problem:
    """One set of operator inputs, host-resident, in the operator's layouts."""

    name: str
    m: int
    k: int
    n: int
    e: int
    x1: np.ndarray                       # int8 (m,k)
    x2: np.ndarray                       # int8 (e,k,n) or int32 (e,k,n/8)
    x2_int4: bool                        # True -> x2 is the packed int4 form
    scale: Optional[np.ndarray]          # float32 or uint16(bf16) (e,1,n)
    scale_bf16: bool
    pertoken_scale: Optional[np.ndarray]  # float32 (m)
    logit: Optional[np.ndarray]          # float32 (m)
    group_list: np.ndarray               # int64 (e)
    group_list_type: int                 # 0 cumulative, 1 counts
    row_index: Optional[np.ndarray]      # int64 or int32 (m)
    shared_input: Optional[np.ndarray]   # uint16(bf16) (bsdp,n)
    shared_input_offset: int
    output_bs: int
    seed: int = 0
    counts: Optional[np.ndarray] = None  # rows per expert (for statistics)
    x2_transposed: bool = False          # True -> int8 x2 is given as (e,n,k)
    fp8: bool = False                    # FP8 mode: x1 uint8 FP8-E4M3 codes (m,k), x2 uint8 codes (e,n,k);
                                         # scale and pertoken_scale as in the int8 mode
    mx: bool = False                     # MxA8W4: x1 uint8 FP8-E4M3 codes (m,k); x2 uint8 (e,n,k/2)
                                         # FP4-E2M1 pairs (low nibble = even k); pertoken_scale uint8
                                         # E8M0 (m,k/64,2); scale uint8 E8M0 (e,n,k/64,2)

    @property
    def bsdp(self) -> int:
        return 0 if self.shared_input is None else int(self.shared_input.shape[0])

    @property
    def covered_rows(self) -> int:
        return int(self.counts.sum()) if self.counts is not None else self.m

    @property
    def nonempty_experts(self) -> int:
        return int((self.counts > 0).sum()) if self.counts is not None else self.e


def _group_list(counts: np.ndarray, group_list_type: int) -> np.ndarray:
    counts = np.asarray(counts, dtype=np.int64)
    return np.cumsum(counts).astype(np.int64) if group_list_type == 0 else counts.copy()


def _row_index(rng, T: int, K: int, dtype) -> np.ndarray:
    """Every token receives exactly K rows; rows are laid over the expert-sorted
    order at random, so a (token, expert) pair may repeat."""
    return rng.permutation(np.repeat(np.arange(T, dtype=np.int64), K)).astype(dtype)


def _topk_softmax_logit(rng, T: int, K: int, row_index: np.ndarray, n_gate: int = 256) -> np.ndarray:
    """Routing weights: per token, K largest of n_gate N(0,1) gate scores,
    softmax in float64, stored as fp32; a token's j-th row (ascending row order)
    takes weight j."""
    scores = rng.standard_normal((T, n_gate))
    top = -np.sort(-scores, axis=1)[:, :K]
    w = np.exp(top - top[:, :1])
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    logit = np.empty(row_index.shape[0], dtype=np.float32)
    seen = np.zeros(T, dtype=np.int64)
    ri = row_index.astype(np.int64)
    for i in range(ri.shape[0]):
        t = ri[i]
        logit[i] = w[t, seen[t] % K]
        seen[t] += 1
    return logit


def _largest_remainder(weights: np.ndarray, total: int) -> np.ndarray:
    q = weights / weights.sum() * total
    base = np.floor(q).astype(np.int64)
    rem = total - int(base.sum())
    order = np.argsort(-(q - base), kind="stable")
    base[order[:rem]] += 1
    return base


def _int8(rng, shape, lo, hi) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int8)


# ---------------------------------------------------------------- named configs

CONFIG_NAMES = ("tiny", "decode", "skewed", "prefill", "int4")


def make_config(name: str, seed: int = 0) -> Problem:
    """The five named workloads (sizes from the operator's A2/A3 limits:
    k = 2048, n = 7168, e <= 256, m <= 131072)."""
    rng = np.random.default_rng(seed)
    if name == "tiny":
        T, K, e, k, n, obs = 16, 2, 4, 256, 256, 16
        counts = np.array([8, 8, 8, 8], dtype=np.int64)
        glt = 0
        ri = _row_index(rng, T, K, np.int64)
        logit = rng.uniform(0.0, 1.0, size=T * K).astype(np.float32)
        x1 = _int8(rng, (T * K, k), -8, 7)
        x2 = _int8(rng, (e, k, n), -8, 7)
        scale = rng.uniform(0.5, 1.5, size=(e, 1, n)).astype(np.float32)
        pts = rng.uniform(0.5, 1.5, size=T * K).astype(np.float32)
        return Problem(name, T * K, k, n, e, x1, x2, False, scale, False, pts, logit,
                       _group_list(counts, glt), glt, ri, None, 0, obs, seed, counts)
    if name == "decode":
        T, K, e, k, n, obs = 512, 8, 8, 2048, 7168, 512
        m = T * K
        counts = rng.multinomial(m, np.full(e, 1.0 / e)).astype(np.int64)
        glt = 1
        ri = _row_index(rng, T, K, np.int64)
        logit = _topk_softmax_logit(rng, T, K, ri)
        x1 = _int8(rng, (m, k), -127, 127)
        x2 = _int8(rng, (e, k, n), -127, 127)
        scale = rng.uniform(1e-3, 1e-2, size=(e, 1, n)).astype(np.float32)
        pts = rng.uniform(1e-3, 1e-2, size=m).astype(np.float32)
        shared = f32_to_bf16_bits(rng.standard_normal((obs, n)).astype(np.float32))
        return Problem(name, m, k, n, e, x1, x2, False, scale, False, pts, logit,
                       _group_list(counts, glt), glt, ri, shared, 0, obs, seed, counts)
    if name == "skewed":
        T, K, e, k, n, obs = 256, 8, 256, 2048, 7168, 256
        m = T * K
        ranks = np.arange(1, e + 1, dtype=np.float64)
        p_rank = ranks ** -1.2
        p_rank /= p_rank.sum()
        perm = rng.permutation(e)
        p = np.empty(e)
        p[perm] = p_rank
        counts = rng.multinomial(m, p).astype(np.int64)
        glt = 0
        ri = _row_index(rng, T, K, np.int32)
        logit = _topk_softmax_logit(rng, T, K, ri)
        x1 = _int8(rng, (m, k), -127, 127)
        x2 = _int8(rng, (e, k, n), -127, 127)
        scale = rng.uniform(1e-3, 1e-2, size=(e, 1, n)).astype(np.float32)
        pts = rng.uniform(1e-3, 1e-2, size=m).astype(np.float32)
        return Problem(name, m, k, n, e, x1, x2, False, scale, False, pts, logit,
                       _group_list(counts, glt), glt, ri, None, 0, obs, seed, counts)
    if name == "prefill":
        T, K, e, k, n, obs = 16384, 8, 32, 2048, 7168, 16384
        m = T * K
        u = rng.uniform(-0.2, 0.2, size=e)
        counts = _largest_remainder(4096.0 * (1.0 + u), m)
        glt = 0
        ri = _row_index(rng, T, K, np.int64)
        logit = _topk_softmax_logit(rng, T, K, ri)
        x1 = _int8(rng, (m, k), -127, 127)
        x2 = _int8(rng, (e, k, n), -127, 127)
        scale = f32_to_bf16_bits(rng.uniform(1e-3, 1e-2, size=(e, 1, n)).astype(np.float32))
        pts = rng.uniform(1e-3, 1e-2, size=m).astype(np.float32)
        shared = f32_to_bf16_bits(rng.standard_normal((8192, n)).astype(np.float32))
        return Problem(name, m, k, n, e, x1, x2, False, scale, True, pts, logit,
                       _group_list(counts, glt), glt, ri, shared, 4096, obs, seed, counts)
    if name == "int4":
        T, K, e, k, n, obs = 4096, 8, 64, 2048, 7168, 4096
        m = T * K
        counts = rng.multinomial(m, rng.dirichlet(np.full(e, 0.5))).astype(np.int64)
        glt = 1
        ri = _row_index(rng, T, K, np.int64)
        logit = _topk_softmax_logit(rng, T, K, ri)
        x1 = _int8(rng, (m, k), -127, 127)
        x2 = pack_int4(_int8(rng, (e, k, n), -8, 7))
        scale = rng.uniform(1e-3, 1e-2, size=(e, 1, n)).astype(np.float32)
        pts = rng.uniform(1e-3, 1e-2, size=m).astype(np.float32)
        return Problem(name, m, k, n, e, x1, x2, True, scale, False, pts, logit,
                       _group_list(counts, glt), glt, ri, None, 0, obs, seed, counts)
    raise ValueError(f"unknown config {name!r}; choose from {CONFIG_NAMES}")


# ---------------------------------------------------------------- random small cases


def random_problem(seed: int, m: int, k: int, n: int, e: int, *,
                   int4: bool = False, scale_bf16: bool = False,
                   group_list_type: int = 0, row_index_dtype=np.int64,
                   with_scale: bool = True, with_pts: bool = True,
                   with_logit: bool = True, with_row_index: bool = True,
                   bsdp: int = 0, shared_offset: int = 0, output_bs: Optional[int] = None,
                   empty_frac: float = 0.25, uncovered: int = 0,
                   lo: int = -128, hi: int = 127) -> Problem:
    """A random problem of the given size for parity and invariant tests.

    Rows per expert are random (some experts empty, with probability
    ``empty_frac``); the last ``uncovered`` rows lie outside every group.
    Destinations are uniform in [0, output_bs), so a destination may receive
    any number of rows, including two from the same expert.
    """
    rng = np.random.default_rng(seed)
    covered = m - uncovered
    if covered < 0:
        raise ValueError("uncovered > m")
    w = rng.uniform(0.2, 1.0, size=e) * (rng.uniform(size=e) >= empty_frac)
    if w.sum() == 0:
        w[rng.integers(e)] = 1.0
    counts = _largest_remainder(w, covered) if covered > 0 else np.zeros(e, dtype=np.int64)
    if output_bs is None:
        output_bs = max(1, m // 2)
    ri = rng.integers(0, output_bs, size=m).astype(row_index_dtype) if with_row_index else None
    logit = rng.uniform(0.0, 1.0, size=m).astype(np.float32) if with_logit else None
    x1 = _int8(rng, (m, k), lo, hi)
    if int4:
        x2 = pack_int4(_int8(rng, (e, k, n), -8, 7))
    else:
        x2 = _int8(rng, (e, k, n), lo, hi)
    scale = None
    if with_scale:
        s = rng.uniform(0.25, 2.0, size=(e, 1, n)).astype(np.float32)
        scale = f32_to_bf16_bits(s) if scale_bf16 else s
    pts = rng.uniform(0.25, 2.0, size=m).astype(np.float32) if with_pts else None
    shared = None
    if bsdp > 0:
        shared = f32_to_bf16_bits(rng.standard_normal((bsdp, n)).astype(np.float32) * 64.0)
    return Problem(f"random{seed}", m, k, n, e, x1, x2, int4, scale, scale_bf16 and with_scale,
                   pts, logit, _group_list(counts, group_list_type), group_list_type, ri,
                   shared, shared_offset, output_bs, seed, counts)


def with_transposed_weights(p: Problem) -> Problem:
    """The same problem with its int8 or FP8 weights given transposed, (e,n,k)."""
    if p.x2_int4 or p.x2_transposed or p.mx:
        raise ValueError("transposed weights are taken from an untransposed int8 or FP8 problem")
    return dataclasses.replace(p, x2=np.ascontiguousarray(np.transpose(p.x2, (0, 2, 1))), x2_transposed=True,
                               name=p.name + "-tb")



def with_per_tensor_scale(p: Problem, value: float | None = None) -> Problem:
    """The same problem with one static per-tensor activation scale in place of
    the per-token pertokenScale: its first entry, or ``value``."""
    if value is None:
        value = float(p.pertoken_scale[0]) if p.pertoken_scale is not None and len(p.pertoken_scale) else 0.005
    return dataclasses.replace(p, pertoken_scale=np.array([value], dtype=np.float32), name=p.name + "-pt")


# ---------------------------------------------------------------- MxA8W4 inputs


def _fp8_codes(rng, shape) -> np.ndarray:
    """FP8 E4M3 codes: random sign, exponent field 3..11 (|v| in [2^-4, 2^4 * 1.875]),
    random mantissa, about 1 in 16 set to zero; never the NaN codes 0x7F/0xFF."""
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8) << 7
    ex = rng.integers(3, 12, size=shape, dtype=np.uint8) << 3
    man = rng.integers(0, 8, size=shape, dtype=np.uint8)
    codes = (sign | ex | man).astype(np.uint8)
    codes[rng.uniform(size=shape) < 1.0 / 16] = 0
    return codes


def _fp4_pairs(rng, shape_pairs) -> np.ndarray:
    """Random FP4 E2M1 codes, two per byte (every code is a number)."""
    return rng.integers(0, 256, size=shape_pairs, dtype=np.int64).astype(np.uint8)


def _e8m0(rng, shape, lo=120, hi=134) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.uint8)


def mx_problem(seed: int, m: int, k: int, n: int, e: int, *, group_list_type: int = 0,
               with_logit: bool = True, with_row_index: bool = True, bsdp: int = 0, shared_offset: int = 0,
               output_bs: Optional[int] = None, empty_frac: float = 0.25, uncovered: int = 0) -> Problem:
    """A random MxA8W4 problem (FP8 activations, FP4 weights given (e,n,k), E8M0
    block scales per 32 k) for parity and invariant tests."""
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    rng = np.random.default_rng(seed)
    covered = m - uncovered
    w = rng.uniform(0.2, 1.0, size=e) * (rng.uniform(size=e) >= empty_frac)
    if w.sum() == 0:
        w[rng.integers(e)] = 1.0
    counts = _largest_remainder(w, covered) if covered > 0 else np.zeros(e, dtype=np.int64)
    if output_bs is None:
        output_bs = max(1, m // 2)
    ri = rng.integers(0, output_bs, size=m).astype(np.int64) if with_row_index else None
    logit = rng.uniform(0.0, 1.0, size=m).astype(np.float32) if with_logit else None
    x1 = _fp8_codes(rng, (m, k))
    x2 = _fp4_pairs(rng, (e, n, k // 2))
    # one E8M0 per 32 k, in pairs: (.., ceil(k/64), 2); with k % 64 == 32 the
    # last pair's second byte is no block's scale (drawn like the others)
    pts = _e8m0(rng, (m, (k + 63) // 64, 2))
    scale = _e8m0(rng, (e, n, (k + 63) // 64, 2))
    shared = None
    if bsdp > 0:
        shared = f32_to_bf16_bits(rng.standard_normal((bsdp, n)).astype(np.float32) * 64.0)
    return Problem(f"mx{seed}", m, k, n, e, x1, x2, False, scale, False, pts, logit,
                   _group_list(counts, group_list_type), group_list_type, ri, shared, shared_offset, output_bs,
                   seed, counts, True, mx=True)


def make_mx_config(name: str = "mxa8w4", seed: int = 0) -> Problem:
    """MxA8W4 at the prefill shape: 16384 tokens, top-8, 32 experts, k = 2048,
    n = 7168, routing, logit and sharedInput drawn as for the prefill workload;
    FP8 activations, FP4 weights (e,n,k) and E8M0 block scales drawn uniformly."""
    if name != "mxa8w4":
        raise ValueError(name)
    rng = np.random.default_rng(seed)
    T, K, e, k, n, obs = 16384, 8, 32, 2048, 7168, 16384
    m = T * K
    u = rng.uniform(-0.2, 0.2, size=e)
    counts = _largest_remainder(4096.0 * (1.0 + u), m)
    ri = _row_index(rng, T, K, np.int64)
    logit = _topk_softmax_logit(rng, T, K, ri)
    x1 = _fp8_codes(rng, (m, k))
    x2 = _fp4_pairs(rng, (e, n, k // 2))
    pts = _e8m0(rng, (m, k // 64, 2))
    scale = _e8m0(rng, (e, n, k // 64, 2))
    shared = f32_to_bf16_bits(rng.standard_normal((8192, n)).astype(np.float32))
    return Problem(name, m, k, n, e, x1, x2, False, scale, False, pts, logit,
                   _group_list(counts, 0), 0, ri, shared, 4096, obs, seed, counts, True, mx=True)


def fp8_problem(seed: int, m: int, k: int, n: int, e: int, *, scale_bf16: bool = False, group_list_type: int = 0,
                with_scale: bool = True, with_pts: bool = True, with_logit: bool = True,
                with_row_index: bool = True, bsdp: int = 0, shared_offset: int = 0,
                output_bs: Optional[int] = None, empty_frac: float = 0.25, uncovered: int = 0) -> Problem:
    """A random FP8 problem: FP8 E4M3 activations and weights (e,n,k), fp32 or
    bf16 per-channel scale, fp32 per-token scale."""
    rng = np.random.default_rng(seed)
    covered = m - uncovered
    w = rng.uniform(0.2, 1.0, size=e) * (rng.uniform(size=e) >= empty_frac)
    if w.sum() == 0:
        w[rng.integers(e)] = 1.0
    counts = _largest_remainder(w, covered) if covered > 0 else np.zeros(e, dtype=np.int64)
    if output_bs is None:
        output_bs = max(1, m // 2)
    ri = rng.integers(0, output_bs, size=m).astype(np.int64) if with_row_index else None
    logit = rng.uniform(0.0, 1.0, size=m).astype(np.float32) if with_logit else None
    x1 = _fp8_codes(rng, (m, k))
    x2 = _fp8_codes(rng, (e, n, k))
    scale = None
    if with_scale:
        sc = rng.uniform(0.25, 2.0, size=(e, 1, n)).astype(np.float32)
        scale = f32_to_bf16_bits(sc) if scale_bf16 else sc
    pts = rng.uniform(0.25, 2.0, size=m).astype(np.float32) if with_pts else None
    shared = None
    if bsdp > 0:
        shared = f32_to_bf16_bits(rng.standard_normal((bsdp, n)).astype(np.float32) * 64.0)
    return Problem(f"fp8{seed}", m, k, n, e, x1, x2, False, scale, scale_bf16 and with_scale, pts, logit,
                   _group_list(counts, group_list_type), group_list_type, ri, shared, shared_offset, output_bs,
                   seed, counts, True, fp8=True)


def with_untransposed_fp8_weights(p: Problem) -> Problem:
    """The same FP8 problem with its weights given untransposed, (e,k,n)."""
    if not p.fp8 or not p.x2_transposed:
        raise ValueError("untransposed weights are taken from an FP8 problem with (e,n,k) weights")
    return dataclasses.replace(p, x2=np.ascontiguousarray(np.transpose(p.x2, (0, 2, 1))), x2_transposed=False,
                               name=p.name + "-kn")


def make_fp8_config(name: str = "fp8", seed: int = 0) -> Problem:
    """FP8 E4M3 at the prefill shape: routing, logit, bf16 per-channel scale,
    pertokenScale and sharedInput drawn as for the prefill workload; FP8
    activations and weights drawn like the MxA8W4 activations, the weights
    given untransposed, (e,k,n) (drawn as (e,n,k) codes and transposed)."""
    if name != "fp8":
        raise ValueError(name)
    rng = np.random.default_rng(seed)
    T, K, e, k, n, obs = 16384, 8, 32, 2048, 7168, 16384
    m = T * K
    u = rng.uniform(-0.2, 0.2, size=e)
    counts = _largest_remainder(4096.0 * (1.0 + u), m)
    ri = _row_index(rng, T, K, np.int64)
    logit = _topk_softmax_logit(rng, T, K, ri)
    x1 = _fp8_codes(rng, (m, k))
    x2 = _fp8_codes(rng, (e, n, k))
    scale = f32_to_bf16_bits(rng.uniform(1e-3, 1e-2, size=(e, 1, n)).astype(np.float32))
    pts = rng.uniform(1e-3, 1e-2, size=m).astype(np.float32)
    shared = f32_to_bf16_bits(rng.standard_normal((8192, n)).astype(np.float32))
    p = Problem(name, m, k, n, e, x1, x2, False, scale, True, pts, logit,
                _group_list(counts, 0), 0, ri, shared, 4096, obs, seed, counts, True, fp8=True)
    return dataclasses.replace(with_untransposed_fp8_weights(p), name=name)


# ---------------------------------------------------------------- activation quant + routing permute inputs


@dataclasses.dataclass
class RouteProblem:
    """Inputs of the step that produces the grouped matmul's inputs: bf16
    hidden states of T tokens and the router's top-K choice per token.

    hidden        uint16 (bf16 bits) (T,k)
    expert_ids    int32 or int64 (T,K): global expert of each (token, slot);
                  local experts are [expert_offset, expert_offset + e)
    topk_weights  float32 (T,K) routing weights, or None
    """

    name: str
    T: int
    k: int
    K: int
    e: int
    hidden: np.ndarray
    expert_ids: np.ndarray
    topk_weights: Optional[np.ndarray]
    expert_offset: int = 0
    group_list_type: int = 1
    seed: int = 0
    mode: str = "int8"   # x1 as int8 per token, "fp8" per token, or "mx" (FP8 with E8M0 per 32 k)

    @property
    def m(self) -> int:
        return self.T * self.K


def route_problem(seed: int, T: int, k: int, K: int, e: int, *, n_gate: Optional[int] = None,
                  expert_offset: int = 0, ids_dtype=np.int64, with_weights: bool = True,
                  group_list_type: int = 1, zero_tokens: int = 0, repeat_slots: bool = False) -> RouteProblem:
    """Seeded router outputs and hidden states.  Draw order: gate scores ->
    hidden.  Gate scores N(0,1) over n_gate experts (default e + expert_offset,
    so every id below expert_offset belongs to another rank); each token takes
    its K largest, with softmax weights (float64, stored fp32).  Hidden values
    are N(0,1) times a per-token magnitude 2^U(-4,4), rounded to bf16; the
    first ``zero_tokens`` tokens are all zero.  ``repeat_slots`` gives every
    token's last slot the expert of its first (a repeated expert)."""
    rng = np.random.default_rng(seed)
    n_gate = e + expert_offset if n_gate is None else n_gate
    if K > n_gate:
        raise ValueError("K exceeds the number of gate experts")
    scores = rng.standard_normal((T, n_gate))
    ids = np.argsort(-scores, axis=1, kind="stable")[:, :K]
    top = np.take_along_axis(scores, ids, axis=1)
    w = np.exp(top - top[:, :1]) if K > 0 else top
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32) if K > 0 else w.astype(np.float32)
    if repeat_slots and K > 1:
        ids[:, K - 1] = ids[:, 0]
    mag = np.exp2(rng.uniform(-4.0, 4.0, size=(T, 1)))
    hidden = (rng.standard_normal((T, k)) * mag).astype(np.float32)
    hidden[:zero_tokens] = 0.0
    return RouteProblem(f"route{seed}", T, k, K, e, f32_to_bf16_bits(hidden), ids.astype(ids_dtype),
                        w if with_weights else None, expert_offset, group_list_type, seed)


def make_route_config(name: str = "dispatch", seed: int = 0) -> RouteProblem:
    """The prefill workload's producer step: 16384 tokens of hidden size 2048,
    top-8 of 32 experts (131072 rows), int64 ids, counts as groupList."""
    if name != "dispatch":
        raise ValueError(name)
    return route_problem(seed, 16384, 2048, 8, 32, ids_dtype=np.int64, group_list_type=1)
