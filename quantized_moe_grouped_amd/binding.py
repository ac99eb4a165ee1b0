"""ctypes binding of libgmmfr.so -- argument marshalling only.

Every step of the computation runs in the HIP library; this module turns torch
tensors into the C descriptors of include/gmmfr.h and forwards the current HIP
stream.  It raises when the library is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgmmfr.so")

# status codes (gmmfr_status)
OK, ERR_NULLPTR, ERR_DTYPE, ERR_SHAPE, ERR_ATTR, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP = range(9)
STATUS_NAMES = {0: "OK", 1: "NULLPTR", 2: "DTYPE", 3: "SHAPE", 4: "ATTR", 5: "UNSUPPORTED", 6: "ALIGN",
                7: "WORKSPACE", 8: "HIP"}
# element types (gmmfr_dtype)
DT_NONE, DT_INT8, DT_INT4, DT_INT32, DT_INT64, DT_FLOAT32, DT_BFLOAT16 = range(7)
DT_FLOAT8_E4M3FN, DT_FLOAT4_E2M1X2, DT_FLOAT8_E8M0 = 7, 8, 9
COMBINE = {"auto": 0, "atomic": 1, "ordered": 2}
COMBINE_HYBRID = 3  # reported by the plan only

EXPORTED = ("gmm_finalize_routing_workspace", "gmm_finalize_routing", "gmm_finalize_routing_profiled",
            "gmm_finalize_routing_plan", "gmmfr_status_string", "gmm_quant_permute_workspace",
            "gmm_quant_permute", "gmm_quant_permute_profiled", "gmm_finalize_routing_noalloc")
NOALLOC_SCRATCH_BYTES = 128 << 20  # GMMFR_NOALLOC_SCRATCH_BYTES


class GmmfrError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        self.status = STATUS_NAMES.get(code, str(code))
        super().__init__(f"{where}: {self.status}")


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("dims", ctypes.c_int64 * 4)]


class Args(ctypes.Structure):
    _fields_ = [
        ("x1", Tensor), ("x2", Tensor), ("scale", Tensor),
        ("bias", Tensor), ("offset", Tensor), ("antiquant_scale", Tensor), ("antiquant_offset", Tensor),
        ("pertoken_scale", Tensor), ("group_list", Tensor), ("shared_input", Tensor), ("logit", Tensor),
        ("row_index", Tensor), ("out", Tensor), ("acc_out", Tensor),
        ("group_list_type", ctypes.c_int64), ("shared_input_offset", ctypes.c_int64), ("output_bs", ctypes.c_int64),
        ("transpose_x1", ctypes.c_int32), ("transpose_x2", ctypes.c_int32),
        ("deterministic", ctypes.c_int32), ("combine", ctypes.c_int32),
        ("tuning_config", ctypes.POINTER(ctypes.c_int64)), ("tuning_config_len", ctypes.c_int64),
    ]


class QpArgs(ctypes.Structure):
    _fields_ = [
        ("hidden", Tensor), ("expert_ids", Tensor), ("topk_weights", Tensor), ("x1", Tensor),
        ("pertoken_scale", Tensor), ("logit", Tensor), ("row_index", Tensor), ("group_list", Tensor),
        ("expert_offset", ctypes.c_int64), ("group_list_type", ctypes.c_int64),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [("combine", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_k", ctypes.c_int32), ("grid", ctypes.c_int32), ("int4_weights", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64), ("gemm_kernel", ctypes.c_char * 96),
                ("hybrid_atomic", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library; raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m quantized_moe_grouped_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.gmm_finalize_routing_workspace.argtypes = [ctypes.POINTER(Args), ctypes.POINTER(ctypes.c_size_t)]
        L.gmm_finalize_routing_workspace.restype = ctypes.c_int
        L.gmm_finalize_routing.argtypes = [ctypes.POINTER(Args), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.gmm_finalize_routing.restype = ctypes.c_int
        L.gmm_finalize_routing_profiled.argtypes = [ctypes.POINTER(Args), ctypes.c_void_p, ctypes.c_size_t,
                                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.gmm_finalize_routing_profiled.restype = ctypes.c_int
        L.gmm_finalize_routing_noalloc.argtypes = [ctypes.POINTER(Args), ctypes.c_void_p]
        L.gmm_finalize_routing_noalloc.restype = ctypes.c_int
        L.gmm_finalize_routing_plan.argtypes = [ctypes.POINTER(Args), ctypes.POINTER(PlanInfo)]
        L.gmm_finalize_routing_plan.restype = ctypes.c_int
        L.gmm_quant_permute_workspace.argtypes = [ctypes.POINTER(QpArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.gmm_quant_permute_workspace.restype = ctypes.c_int
        L.gmm_quant_permute.argtypes = [ctypes.POINTER(QpArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.gmm_quant_permute.restype = ctypes.c_int
        L.gmm_quant_permute_profiled.argtypes = [ctypes.POINTER(QpArgs), ctypes.c_void_p, ctypes.c_size_t,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.gmm_quant_permute_profiled.restype = ctypes.c_int
        L.gmmfr_status_string.argtypes = [ctypes.c_int]
        L.gmmfr_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _dtype_code(t, int4_packed: bool = False) -> int:
    import torch
    if t.dtype == torch.int8:
        return DT_INT8
    if t.dtype == torch.int32:
        return DT_INT32
    if t.dtype == torch.int64:
        return DT_INT64
    if t.dtype == torch.float32:
        return DT_FLOAT32
    if t.dtype == torch.bfloat16:
        return DT_BFLOAT16
    if t.dtype == torch.float8_e4m3fn:
        return DT_FLOAT8_E4M3FN
    if t.dtype == torch.float4_e2m1fn_x2:
        return DT_FLOAT4_E2M1X2
    if t.dtype == torch.float8_e8m0fnu:
        return DT_FLOAT8_E8M0
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _desc(t, dtype: Optional[int] = None) -> Tensor:
    d = Tensor()
    if t is None:
        return d
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if t.dim() > 4:
        raise ValueError("at most 4 dimensions")
    d.data = t.data_ptr()
    d.dtype = _dtype_code(t) if dtype is None else dtype
    d.ndim = t.dim()
    for i, s in enumerate(t.shape):
        d.dims[i] = int(s)
    return d


def make_args(x1, x2, group_list, out, *, scale=None, pertoken_scale=None, logit=None, row_index=None,
              shared_input=None, shared_input_offset: int = 0, group_list_type: int = 0,
              deterministic: bool = False, combine: str = "auto", acc_out=None,
              tuning_config: Optional[Sequence[int]] = None, bias=None, offset=None,
              antiquant_scale=None, antiquant_offset=None, transpose_x1: bool = False,
              transpose_x2: bool = False):
    """Build the C argument struct.  Returns (args, keepalive): the struct holds
    raw device pointers, so keep `keepalive` (which references every tensor
    passed, and the host tuning array) alive until the call has been enqueued
    and the stream has reached it."""
    a = Args()
    a.x1 = _desc(x1)
    a.x2 = _desc(x2)
    a.scale = _desc(scale)
    a.bias = _desc(bias)
    a.offset = _desc(offset)
    a.antiquant_scale = _desc(antiquant_scale)
    a.antiquant_offset = _desc(antiquant_offset)
    a.pertoken_scale = _desc(pertoken_scale)
    a.group_list = _desc(group_list)
    a.shared_input = _desc(shared_input)
    a.logit = _desc(logit)
    a.row_index = _desc(row_index)
    a.out = _desc(out)
    a.acc_out = _desc(acc_out)
    a.group_list_type = int(group_list_type)
    a.shared_input_offset = int(shared_input_offset)
    a.output_bs = int(out.shape[0]) if out is not None else 0
    a.transpose_x1 = int(bool(transpose_x1))
    a.transpose_x2 = int(bool(transpose_x2))
    a.deterministic = int(bool(deterministic))
    a.combine = COMBINE[combine]
    tuning = None
    if tuning_config:
        tuning = (ctypes.c_int64 * len(tuning_config))(*[int(v) for v in tuning_config])
        a.tuning_config = ctypes.cast(tuning, ctypes.POINTER(ctypes.c_int64))
        a.tuning_config_len = len(tuning_config)
    keep = (x1, x2, group_list, out, scale, pertoken_scale, logit, row_index, shared_input, acc_out, bias, offset,
            antiquant_scale, antiquant_offset, tuning)
    return a, keep


def workspace_size(args: Args) -> int:
    n = ctypes.c_size_t(0)
    st = lib().gmm_finalize_routing_workspace(ctypes.byref(args), ctypes.byref(n))
    if st != OK:
        raise GmmfrError(st, "gmm_finalize_routing_workspace")
    return int(n.value)


def plan(args: Args) -> dict:
    info = PlanInfo()
    st = lib().gmm_finalize_routing_plan(ctypes.byref(args), ctypes.byref(info))
    if st != OK:
        raise GmmfrError(st, "gmm_finalize_routing_plan")
    return {"combine": {1: "atomic", 2: "ordered", 3: "hybrid"}[info.combine], "tile_m": info.tile_m,
            "tile_n": info.tile_n, "tile_k": info.tile_k, "grid": info.grid, "int4_weights": bool(info.int4_weights),
            "workspace_bytes": int(info.workspace_bytes), "gemm_kernel": info.gemm_kernel.decode(),
            "hybrid_atomic": int(info.hybrid_atomic)}


def _torch_stream(stream):
    """The torch stream object for `stream`: None (the current stream), a
    torch.cuda.Stream, or a raw hipStream_t handle."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    if int(stream) == 0:  # the null stream
        return torch.cuda.default_stream()
    return torch.cuda.ExternalStream(int(stream))


def run(args: Args, workspace=None, stream=None) -> None:
    """Enqueue on `stream` (default: torch's current stream on the current device)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    ws_ptr = 0 if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().gmm_finalize_routing(ctypes.byref(args), ctypes.c_void_p(ws_ptr), ctypes.c_size_t(ws_bytes),
                                    ctypes.c_void_p(stream))
    if st != OK:
        raise GmmfrError(st, "gmm_finalize_routing")


def gmm_finalize_routing(x1, x2, group_list, out, *, workspace=None, stream=None, **kw) -> None:
    """One call: validate, size the workspace, allocate it with torch if none
    is given, enqueue.  Keyword arguments are those of make_args.

    A workspace allocated here is taken from the pool of the stream the kernels
    run on, so when it is released on return the caching allocator hands the
    block out again only to work ordered after them on that stream (a block
    from another stream's pool could be reused, and overwritten, while the
    kernels still run)."""
    import torch
    args, keep = make_args(x1, x2, group_list, out, **kw)
    need = workspace_size(args)
    ts = _torch_stream(stream)
    if need and workspace is None:
        with torch.cuda.stream(ts):
            workspace = torch.empty(need, dtype=torch.uint8, device=out.device)
    run(args, workspace, ts)
    del keep


def run_noalloc(args: Args, stream=None) -> None:
    """Enqueue through the allocation-free entry point (the library's own
    scratch array; nothing is allocated) on `stream` (default: the current
    stream)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    st = lib().gmm_finalize_routing_noalloc(ctypes.byref(args), ctypes.c_void_p(stream))
    if st != OK:
        raise GmmfrError(st, "gmm_finalize_routing_noalloc")


def gmm_finalize_routing_noalloc(x1, x2, group_list, out, *, stream=None, **kw) -> None:
    """gmm_finalize_routing without any allocation (see run_noalloc).
    Keyword arguments are those of make_args."""
    args, keep = make_args(x1, x2, group_list, out, **kw)
    run_noalloc(args, stream)
    del keep


# ---------------------------------------------------------------- producer step


def make_qp_args(hidden, expert_ids, x1, pertoken_scale, row_index, group_list, *, topk_weights=None,
                 logit=None, expert_offset: int = 0, group_list_type: int = 1):
    """C arguments of gmm_quant_permute.  hidden is bf16 (T,k) and expert_ids
    int32/int64 (T,K); the outputs are x1 int8 (T*K,k), pertoken_scale fp32
    (T*K), row_index int32/int64 (T*K), group_list int64 (e), and logit fp32
    (T*K) when topk_weights (T,K) is given.  Returns (args, keepalive)."""
    a = QpArgs()
    a.hidden = _desc(hidden)
    a.expert_ids = _desc(expert_ids)
    a.topk_weights = _desc(topk_weights)
    a.x1 = _desc(x1)
    a.pertoken_scale = _desc(pertoken_scale)
    a.logit = _desc(logit)
    a.row_index = _desc(row_index)
    a.group_list = _desc(group_list)
    a.expert_offset = int(expert_offset)
    a.group_list_type = int(group_list_type)
    return a, (hidden, expert_ids, topk_weights, x1, pertoken_scale, logit, row_index, group_list)


def qp_workspace_size(args: QpArgs) -> int:
    n = ctypes.c_size_t(0)
    st = lib().gmm_quant_permute_workspace(ctypes.byref(args), ctypes.byref(n))
    if st != OK:
        raise GmmfrError(st, "gmm_quant_permute_workspace")
    return int(n.value)


def quant_permute(hidden, expert_ids, num_experts: int, *, topk_weights=None, expert_offset: int = 0,
                  group_list_type: int = 1, row_index_dtype=None, mode: str = "int8", workspace=None,
                  stream=None) -> dict:
    """Allocate the outputs with torch and enqueue gmm_quant_permute on `stream`
    (default: the current stream).  mode: "int8" (int8 x1, fp32 per-token
    scale), "fp8" (FP8 E4M3 x1, fp32 per-token scale) or "mx" (FP8 E4M3 x1,
    E8M0 scale per 32 values, (m, k/64, 2)).  Returns the output tensors by name."""
    import torch
    dev = hidden.device
    T, k = hidden.shape
    K = expert_ids.shape[1]
    m = T * K
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):  # outputs and workspace from the pool of the stream that writes them
        return _quant_permute_on(hidden, expert_ids, num_experts, topk_weights, expert_offset, group_list_type,
                                 row_index_dtype, mode, workspace, ts, dev, T, k, m)


def _quant_permute_on(hidden, expert_ids, num_experts, topk_weights, expert_offset, group_list_type,
                      row_index_dtype, mode, workspace, ts, dev, T, k, m):
    import torch
    if mode == "int8":
        x1 = torch.empty((m, k), dtype=torch.int8, device=dev)
        pts = torch.empty(m, dtype=torch.float32, device=dev)
    elif mode == "fp8":
        x1 = torch.empty((m, k), dtype=torch.float8_e4m3fn, device=dev)
        pts = torch.empty(m, dtype=torch.float32, device=dev)
    elif mode == "mx":
        x1 = torch.empty((m, k), dtype=torch.float8_e4m3fn, device=dev)
        pts = torch.empty((m, k // 64, 2), dtype=torch.float8_e8m0fnu, device=dev)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    out = dict(x1=x1,
               pertoken_scale=pts,
               row_index=torch.empty(m, dtype=row_index_dtype or torch.int64, device=dev),
               group_list=torch.empty(num_experts, dtype=torch.int64, device=dev),
               logit=None if topk_weights is None else torch.empty(m, dtype=torch.float32, device=dev))
    args, keep = make_qp_args(hidden, expert_ids, out["x1"], out["pertoken_scale"], out["row_index"],
                              out["group_list"], topk_weights=topk_weights, logit=out["logit"],
                              expert_offset=expert_offset, group_list_type=group_list_type)
    need = qp_workspace_size(args)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = ts.cuda_stream
    ws_ptr = 0 if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().gmm_quant_permute(ctypes.byref(args), ctypes.c_void_p(ws_ptr), ctypes.c_size_t(ws_bytes),
                                 ctypes.c_void_p(stream))
    if st != OK:
        raise GmmfrError(st, "gmm_quant_permute")
    del keep
    out["workspace"] = workspace
    return out
