"""CPU oracle for the grouped quantized MoE matmul + finalize-routing combine.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this package.  It shares no code with
the GPU library: the C oracle (gmmfr_oracle.c) is compiled with gcc on its own,
and the pure-Python brute force (brute.py) is a second, independent reading.

Entry points take any object with the fields of
``quantized_moe_grouped_amd.workloads.Problem`` (duck-typed, nothing imported).

Transposed weights ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2", parameter
notes: x2 is (e,k,n), or (e,n,k) when transposed): int8 x2 given as (e,n,k)
means W_g = x2[g] transposed; the wrapper transposes it back with numpy and the
C oracle computes from W as for untransposed weights.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

ORC_NONE, ORC_I8, ORC_I32, ORC_I64, ORC_F32, ORC_BF16, ORC_I4PACKED = range(7)
STATUS = {0: "OK", 1: "NULL", 2: "DTYPE", 3: "SHAPE", 4: "GROUPLIST", 5: "ROWINDEX", 6: "SHARED"}


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle rejected the inputs: {STATUS.get(code, code)}")
        self.code = code
        self.status = STATUS.get(code, str(code))


class _Problem(ctypes.Structure):
    _fields_ = [
        ("m", ctypes.c_int64), ("k", ctypes.c_int64), ("n", ctypes.c_int64), ("e", ctypes.c_int64),
        ("x1", ctypes.c_void_p),
        ("x2", ctypes.c_void_p), ("x2_type", ctypes.c_int32),
        ("scale", ctypes.c_void_p), ("scale_type", ctypes.c_int32),
        ("pertoken_scale", ctypes.c_void_p),
        ("logit", ctypes.c_void_p),
        ("group_list", ctypes.c_void_p),
        ("group_list_type", ctypes.c_int64),
        ("row_index", ctypes.c_void_p), ("row_index_type", ctypes.c_int32),
        ("shared_input", ctypes.c_void_p),
        ("bsdp", ctypes.c_int64),
        ("shared_input_offset", ctypes.c_int64),
        ("output_bs", ctypes.c_int64),
        ("pertoken_per_tensor", ctypes.c_int32),
    ]


_lib = None


def load():
    """Load liboracle.so, building it first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(LIB_PATH)
        for name in ("orc_gmm_finalize_routing", "orc_out_rows", "orc_acc_rows", "orc_group_ranges"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c_problem(p, keep):
    """Marshal a Problem into the C struct; ``keep`` holds the arrays alive."""
    def arr(a, dtype):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=dtype)
        keep.append(a)
        return a

    x1 = arr(p.x1, np.int8)
    if getattr(p, "x2_transposed", False):
        if p.x2_int4:
            raise OracleError(2)
        x2 = arr(np.transpose(np.asarray(p.x2), (0, 2, 1)), np.int8)  # (e,n,k) -> W (e,k,n)
    else:
        x2 = arr(p.x2, np.int32 if p.x2_int4 else np.int8)
    scale = None
    if p.scale is not None:
        scale = arr(p.scale, np.uint16 if p.scale_bf16 else np.float32)
    pts = arr(p.pertoken_scale, np.float32)
    # pertokenScale (m) per token, or (1): one static per-tensor scale
    if pts is not None and pts.shape != (int(p.m),) and pts.shape != (1,):
        raise OracleError(3)
    logit = arr(p.logit, np.float32)
    gl = arr(p.group_list, np.int64)
    ri = None
    ri_type = ORC_NONE
    if p.row_index is not None:
        ri_type = ORC_I32 if np.asarray(p.row_index).dtype == np.int32 else ORC_I64
        ri = arr(p.row_index, np.int32 if ri_type == ORC_I32 else np.int64)
    shared = arr(p.shared_input, np.uint16)
    c = _Problem()
    c.m, c.k, c.n, c.e = int(p.m), int(p.k), int(p.n), int(p.e)
    c.x1 = _ptr(x1)
    c.x2 = _ptr(x2)
    c.x2_type = ORC_I4PACKED if p.x2_int4 else ORC_I8
    c.scale = _ptr(scale)
    c.scale_type = (ORC_BF16 if p.scale_bf16 else ORC_F32) if scale is not None else ORC_NONE
    c.pertoken_scale = _ptr(pts)
    c.pertoken_per_tensor = int(pts is not None and pts.shape == (1,))
    c.logit = _ptr(logit)
    c.group_list = _ptr(gl)
    c.group_list_type = int(p.group_list_type)
    c.row_index = _ptr(ri)
    c.row_index_type = ri_type
    c.shared_input = _ptr(shared)
    c.bsdp = 0 if shared is None else int(shared.shape[0])
    c.shared_input_offset = int(p.shared_input_offset)
    c.output_bs = int(p.output_bs)
    return c


def run(p, want_acc: bool = True):
    """Whole computation.  Returns (out fp32 (outputBS,n), acc int32 (m,n) or None)."""
    lib = load()
    keep = []
    c = _c_problem(p, keep)
    out = np.empty((int(p.output_bs), int(p.n)), dtype=np.float32)
    acc = np.empty((int(p.m), int(p.n)), dtype=np.int32) if want_acc else None
    st = lib.orc_gmm_finalize_routing(ctypes.byref(c), _ptr(out), _ptr(acc))
    if st != 0:
        raise OracleError(st)
    return out, acc


def out_rows(p, d_list):
    """Output rows d_list (count x n) evaluated from the definition, one by one."""
    lib = load()
    keep = []
    c = _c_problem(p, keep)
    d = np.ascontiguousarray(d_list, dtype=np.int64)
    res = np.empty((d.shape[0], int(p.n)), dtype=np.float32)
    st = lib.orc_out_rows(ctypes.byref(c), ctypes.c_int64(d.shape[0]), _ptr(d), _ptr(res))
    if st != 0:
        raise OracleError(st)
    return res


def acc_rows(p, i_list):
    """int32 accumulators of source rows i_list (count x n)."""
    lib = load()
    keep = []
    c = _c_problem(p, keep)
    i = np.ascontiguousarray(i_list, dtype=np.int64)
    res = np.empty((i.shape[0], int(p.n)), dtype=np.int32)
    st = lib.orc_acc_rows(ctypes.byref(c), ctypes.c_int64(i.shape[0]), _ptr(i), _ptr(res))
    if st != 0:
        raise OracleError(st)
    return res


def group_ranges(p):
    """[start_g, end_g) per expert as two int64 arrays."""
    lib = load()
    keep = []
    c = _c_problem(p, keep)
    s = np.empty(int(p.e), dtype=np.int64)
    e = np.empty(int(p.e), dtype=np.int64)
    st = lib.orc_group_ranges(ctypes.byref(c), _ptr(s), _ptr(e))
    if st != 0:
        raise OracleError(st)
    return s, e


def clamped_ends(group_list, group_list_type: int, m: int):
    """End row of every group under the library's reading of a groupList that
    breaks the operator's rule ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2",
    common constraints: type 0 lists non-negative, non-decreasing cumulative
    ends; type 1 non-negative counts; and the rows they cover lie in x1).  The
    library header states the reading for device data it cannot check: each
    entry is clamped to [0, m]; type 0 ends are the running maximum of the
    clamped entries, type 1 ends the running sum of the clamped counts, capped
    at m.  For a list that keeps the rule this is the plain reading."""
    ends = []
    end = 0
    for x in (int(v) for v in group_list):
        c = min(max(x, 0), int(m))
        end = max(end, c) if int(group_list_type) == 0 else min(end + c, int(m))
        ends.append(end)
    return np.array(ends, dtype=np.int64)


def clamped_problem(p):
    """A problem that keeps every rule and computes what the library computes
    for ``p`` under the clamped reading of its device data: groups end at
    ``clamped_ends`` (given as a type-0 list), and a row whose rowIndex lies
    outside [0, outputBS) contributes nothing -- it is sent to one extra
    destination row outputBS, which the caller drops from the result.
    Returns (problem, rows of the real output)."""
    import copy
    q = copy.copy(p)
    q.group_list = clamped_ends(p.group_list, p.group_list_type, p.m)
    q.group_list_type = 0
    if p.row_index is not None:
        ri = np.asarray(p.row_index).astype(np.int64)
        bad = (ri < 0) | (ri >= int(p.output_bs))
        ri = np.where(bad, int(p.output_bs), ri)
        q.row_index = ri.astype(np.asarray(p.row_index).dtype)
    q.output_bs = int(p.output_bs) + 1
    return q, int(p.output_bs)
