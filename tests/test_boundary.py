"""C-ABI boundary on the CPU: the library loads, exports every function the
header declares, and the first stage validates arguments without touching a
device (pointers here are fake, aligned, never dereferenced)."""
import ctypes
import os
import re

import pytest

from quantized_moe_grouped_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\([^;{]*\)\s*;", text, flags=re.M)
    return names


def test_library_exports_every_declared_function():
    lib = B.lib()
    declared = _declared_functions()
    assert set(B.EXPORTED) <= set(declared)
    for name in declared:
        assert hasattr(lib, name), name


# ---------------------------------------------------------------- fake descriptors

_next = [0x10000]


def _fake(dtype, *dims, ptr=None):
    t = B.Tensor()
    if ptr is None:
        _next[0] += 0x100000
        ptr = _next[0]
    t.data = ptr
    t.dtype = dtype
    t.ndim = len(dims)
    for i, d in enumerate(dims):
        t.dims[i] = d
    return t


def _args(m=512, k=2048, n=7168, e=8, obs=256, int4=False, **over):
    a = B.Args()
    a.x1 = _fake(B.DT_INT8, m, k)
    a.x2 = _fake(B.DT_INT32, e, k, n // 8) if int4 else _fake(B.DT_INT8, e, k, n)
    a.scale = _fake(B.DT_FLOAT32, e, 1, n)
    a.pertoken_scale = _fake(B.DT_FLOAT32, m)
    a.group_list = _fake(B.DT_INT64, e)
    a.logit = _fake(B.DT_FLOAT32, m)
    a.row_index = _fake(B.DT_INT64, m)
    a.out = _fake(B.DT_FLOAT32, obs, n)
    a.output_bs = obs
    for key, v in over.items():
        setattr(a, key, v)
    return a


def _ws(a):
    n = ctypes.c_size_t(12345)
    st = B.lib().gmm_finalize_routing_workspace(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


def test_atomic_workspace_is_the_control_block():
    a = _args(m=32, k=256, n=256, e=4, obs=16)
    a.combine = B.COMBINE["atomic"]
    assert _ws(a) == (B.OK, 1024)


def test_ordered_workspace_formula():
    m, n, obs = 4096, 7168, 512
    a = _args(m=m, n=n, obs=obs)
    a.deterministic = 1

    def al(x):
        return (x + 255) // 256 * 256
    want = 1024 + al(m * n * 4) + al(obs * 4) * 2 + al((obs + 1) * 4) + al(m * 4)
    assert _ws(a) == (B.OK, want)


def test_auto_picks_ordered_for_large_problems():
    a = _args(m=131072, n=7168, obs=16384, e=32)
    info = B.PlanInfo()
    assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.OK
    assert info.combine == B.COMBINE["ordered"]
    assert info.tile_m == 256


@pytest.mark.parametrize("k,int4,want_k,want_name", [
    (2048, False, 128, "gmm_kernel<256,256,128,4x2,s2,i8,cont>"),  # 128 k per stage, two stages
    (512, False, 128, "gmm_kernel<256,256,128,4x2,s2,i8,cont>"),
    (128, False, 128, "gmm_kernel<256,256,128,4x2,s2,i8>"),        # one k-step: tile by tile
    (192, False, 64, "gmm_kernel<256,256,64,4x2,s4,i8>"),          # k % 128 != 0: 64 k, four stages
    (448, False, 64, "gmm_kernel<256,256,64,4x2,s4,i8,cont>"),
    (2048, True, 64, "gmm_kernel<256,256,64,4x2,s4,i4,cont>"),     # int4 weights: 64 k
])
def test_256_row_tile_stage_depth(k, int4, want_k, want_name):
    a = _args(m=8192, k=k, e=4, obs=1024, int4=int4)
    tc = (ctypes.c_int64 * 2)(0, 256)
    a.tuning_config = ctypes.cast(tc, ctypes.POINTER(ctypes.c_int64))
    a.tuning_config_len = 2
    info = B.PlanInfo()
    assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.OK
    assert (info.tile_m, info.tile_n, info.tile_k) == (256, 256, want_k)
    assert info.gemm_kernel.decode() == want_name


@pytest.mark.parametrize("m,e,int4,want", [
    (131072, 32, False, 256),   # prefill-sized experts, int8 weights: the eight-wave 256-row tile
    (131072, 32, True, 128),    # int4 weights keep the 128-row tile
    (4096, 8, False, 128),      # 512-row experts: too few 256-row tiles for the CUs
    (2048, 256, False, 32),     # a few rows per expert
])
def test_auto_tile_follows_the_shape(m, e, int4, want):
    a = _args(m=m, e=e, obs=max(m // 8, 1), int4=int4)
    info = B.PlanInfo()
    assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.OK
    assert info.tile_m == want


@pytest.mark.parametrize("m,e,int4,want", [
    (131072, 32, False, "ordered"),   # prefill-shaped: atomics would outlast the GEMM
    (4096, 8, False, "ordered"),      # decode-shaped
    (32768, 64, True, "ordered"),     # int4 weights: the atomics would reach half the GEMM time
    (2048, 256, False, "atomic"),     # many experts: weight streaming dominates
    (32, 4, False, "atomic"),
])
def test_auto_combine_follows_the_shape(m, e, int4, want):
    a = _args(m=m, e=e, obs=max(m // 8, 1), int4=int4)
    info = B.PlanInfo()
    assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.OK
    assert info.combine == B.COMBINE[want]
    a.deterministic = 1
    assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.OK
    assert info.combine == B.COMBINE["ordered"]


def test_plan_does_not_depend_on_data_and_follows_hint():
    a = _args(m=4096, n=7168, obs=512, e=8)
    info = B.PlanInfo()
    B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info))
    base = info.tile_m
    hint = (ctypes.c_int64 * 1)(8)
    a.tuning_config = ctypes.cast(hint, ctypes.POINTER(ctypes.c_int64))
    a.tuning_config_len = 1
    B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info))
    assert info.tile_m == 32 and base != 32
    for forced in (256, 128, 64, 32):
        hint2 = (ctypes.c_int64 * 2)(0, forced)
        a.tuning_config = ctypes.cast(hint2, ctypes.POINTER(ctypes.c_int64))
        a.tuning_config_len = 2
        assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.OK
        assert info.tile_m == forced
    hint2 = (ctypes.c_int64 * 2)(0, 96)
    a.tuning_config = ctypes.cast(hint2, ctypes.POINTER(ctypes.c_int64))
    assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.ERR_ATTR


@pytest.mark.parametrize("cap", [1, 3, 8, 16, 100000])
def test_grid_cap_limits_the_gemm_launch(cap):
    """tuningConfig[2] caps the persistent GEMM's workgroups (a test hook:
    results do not depend on it); 0 means no cap, negative is rejected."""
    a = _args(m=131072, n=7168, obs=16384, e=32)
    info = B.PlanInfo()
    assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.OK
    full = info.grid
    ws_full = info.workspace_bytes
    hint = (ctypes.c_int64 * 3)(0, 0, cap)
    a.tuning_config = ctypes.cast(hint, ctypes.POINTER(ctypes.c_int64))
    a.tuning_config_len = 3
    assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.OK
    assert info.grid == min(cap, full)
    assert info.workspace_bytes == ws_full
    for bad in (-1, -100):
        hint = (ctypes.c_int64 * 3)(0, 0, bad)
        a.tuning_config = ctypes.cast(hint, ctypes.POINTER(ctypes.c_int64))
        assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.ERR_ATTR
    hint = (ctypes.c_int64 * 3)(0, 0, 0)
    a.tuning_config = ctypes.cast(hint, ctypes.POINTER(ctypes.c_int64))
    assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.OK
    assert info.grid == full


CASES = [
    ("nullptr_x1", dict(x1=B.Tensor()), B.ERR_NULLPTR),
    ("nullptr_group_list", dict(group_list=B.Tensor()), B.ERR_NULLPTR),
    ("nullptr_out", dict(out=B.Tensor()), B.ERR_NULLPTR),
    ("bias_reserved", dict(bias=_fake(B.DT_FLOAT32, 8, 7168)), B.ERR_UNSUPPORTED),
    ("offset_reserved", dict(offset=_fake(B.DT_FLOAT32, 8, 1, 7168)), B.ERR_UNSUPPORTED),
    ("antiquant_reserved", dict(antiquant_scale=_fake(B.DT_FLOAT32, 8, 1, 7168)), B.ERR_UNSUPPORTED),
    ("scale_int64", dict(scale=_fake(B.DT_INT64, 8, 1, 7168)), B.ERR_UNSUPPORTED),
    ("x1_dtype", dict(x1=_fake(B.DT_FLOAT32, 512, 2048)), B.ERR_DTYPE),
    ("x2_dtype", dict(x2=_fake(B.DT_BFLOAT16, 8, 2048, 7168)), B.ERR_DTYPE),
    ("group_list_dtype", dict(group_list=_fake(B.DT_INT32, 8)), B.ERR_DTYPE),
    ("row_index_dtype", dict(row_index=_fake(B.DT_FLOAT32, 512)), B.ERR_DTYPE),
    ("shared_dtype", dict(shared_input=_fake(B.DT_FLOAT32, 128, 7168)), B.ERR_DTYPE),
    ("out_dtype", dict(out=_fake(B.DT_BFLOAT16, 256, 7168)), B.ERR_DTYPE),
    ("group_list_type", dict(group_list_type=2), B.ERR_ATTR),
    ("transpose_x2_value", dict(transpose_x2=2), B.ERR_ATTR),
    ("transpose_x2_int4", dict(transpose_x2=1, x2=_fake(B.DT_INT32, 8, 7168, 256)), B.ERR_UNSUPPORTED),
    ("transpose_x2_k_mismatch", dict(transpose_x2=1, x2=_fake(B.DT_INT8, 8, 7168, 1024)), B.ERR_SHAPE),
    ("transpose_x2_untransposed_dims", dict(transpose_x2=1), B.ERR_SHAPE),
    ("transpose_x1", dict(transpose_x1=1), B.ERR_ATTR),
    ("det_with_atomic", dict(deterministic=1, combine=1), B.ERR_ATTR),
    ("k_mismatch", dict(x2=_fake(B.DT_INT8, 8, 1024, 7168)), B.ERR_SHAPE),
    ("k_not_mult_64", dict(x1=_fake(B.DT_INT8, 512, 2000), x2=_fake(B.DT_INT8, 8, 2000, 7168)), B.ERR_SHAPE),
    ("n_not_mult_16", dict(x2=_fake(B.DT_INT8, 8, 2048, 7160), scale=B.Tensor(),
                           out=_fake(B.DT_FLOAT32, 256, 7160)), B.ERR_SHAPE),
    ("too_many_experts", dict(x2=_fake(B.DT_INT8, 1025, 2048, 16), scale=B.Tensor(), group_list=_fake(B.DT_INT64, 1025),
                              out=_fake(B.DT_FLOAT32, 256, 16)), B.ERR_SHAPE),
    ("scale_shape", dict(scale=_fake(B.DT_FLOAT32, 8, 7168)), B.ERR_SHAPE),
    ("group_list_len", dict(group_list=_fake(B.DT_INT64, 7)), B.ERR_SHAPE),
    ("pts_len", dict(pertoken_scale=_fake(B.DT_FLOAT32, 511)), B.ERR_SHAPE),
    ("pts_len_two", dict(pertoken_scale=_fake(B.DT_FLOAT32, 2)), B.ERR_SHAPE),
    ("out_rows", dict(out=_fake(B.DT_FLOAT32, 255, 7168)), B.ERR_SHAPE),
    ("shared_too_tall", dict(shared_input=_fake(B.DT_BFLOAT16, 257, 7168)), B.ERR_ATTR),
    ("shared_offset", dict(shared_input=_fake(B.DT_BFLOAT16, 128, 7168), shared_input_offset=129), B.ERR_ATTR),
    ("negative_offset", dict(shared_input=_fake(B.DT_BFLOAT16, 128, 7168), shared_input_offset=-1), B.ERR_ATTR),
    ("misaligned", dict(logit=_fake(B.DT_FLOAT32, 512, ptr=0x7000004)), B.ERR_ALIGN),
]


@pytest.mark.parametrize("name,over,code", CASES, ids=[c[0] for c in CASES])
def test_stage_one_rejects(name, over, code):
    a = _args()
    for key, v in over.items():
        setattr(a, key, v)
    st, ws = _ws(a)
    assert st == code, (B.STATUS_NAMES.get(st), B.STATUS_NAMES.get(code))
    assert ws == 12345  # untouched on error


def test_transposed_weights_accepted():
    """x2 (e,n,k) with transpose_x2 = 1 (parameter notes: transposed x2)."""
    a = _args()
    a.transpose_x2 = 1
    a.x2 = _fake(B.DT_INT8, 8, 7168, 2048)
    assert _ws(a)[0] == B.OK
    info = B.PlanInfo()
    assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.OK
    assert info.gemm_kernel.decode().endswith(",tb>")



def test_per_tensor_pertoken_scale_accepted():
    """pertokenScale of shape (1): the static per-tensor activation scale
    (function description: static pertensor-perchannel)."""
    a = _args()
    a.pertoken_scale = _fake(B.DT_FLOAT32, 1)
    assert _ws(a)[0] == B.OK

def test_int4_shapes_accepted_and_checked():
    assert _ws(_args(int4=True))[0] == B.OK
    a = _args(int4=True)
    a.x2 = _fake(B.DT_INT4, 8, 2048, 7168)   # same bytes, logical int4 shape
    assert _ws(a)[0] == B.OK
    a = _args(n=7168 + 16)                    # int8 accepts n % 16 == 0
    assert _ws(a)[0] == B.OK
    a = _args(n=7168 + 16, int4=True)         # int4 needs n % 32 == 0
    assert _ws(a)[0] == B.ERR_SHAPE


def test_zero_rows_accepted():
    assert _ws(_args(m=0))[0] == B.OK


def test_status_strings():
    for code in range(9):
        assert B.lib().gmmfr_status_string(code)
    assert B.lib().gmmfr_status_string(99) == b"unknown status"


def test_stage_two_requires_the_workspace():
    a = _args()
    a.combine = B.COMBINE["atomic"]
    assert B.lib().gmm_finalize_routing(ctypes.byref(a), None, 0, None) == B.ERR_WORKSPACE
    assert B.lib().gmm_finalize_routing(ctypes.byref(a), ctypes.c_void_p(0x100000), 1023, None) == B.ERR_WORKSPACE


def test_stage_two_rejects_before_any_launch():
    """Validation in stage two runs before any HIP call, so a bad argument
    returns its status even on a host without a GPU."""
    a = _args()
    a.group_list_type = 5
    st = B.lib().gmm_finalize_routing(ctypes.byref(a), None, 0, None)
    assert st == B.ERR_ATTR


def test_make_args_keepalive_holds_every_tensor():
    """The argument struct holds raw pointers; the keepalive it comes with must
    keep each tensor passed alive (temporaries included)."""
    import gc
    import weakref
    import torch
    tmp = torch.zeros(16, dtype=torch.int64)
    ref = weakref.ref(tmp)
    x1 = torch.zeros((4, 64), dtype=torch.int8)
    x2 = torch.zeros((1, 64, 16), dtype=torch.int8)
    out = torch.zeros((4, 16), dtype=torch.float32)
    a, keep = B.make_args(x1, x2, torch.tensor([4], dtype=torch.int64), out, row_index=tmp,
                          logit=torch.ones(4, dtype=torch.float32), tuning_config=[0, 64])
    del tmp
    gc.collect()
    assert ref() is not None, "a tensor passed to make_args was freed while its keepalive lives"
    assert a.row_index.data == ref().data_ptr()
    assert any(t is not None and getattr(t, "data_ptr", None) and t.data_ptr() == a.logit.data for t in keep)
    assert a.tuning_config_len == 2 and a.tuning_config[1] == 64
    del keep
    gc.collect()
    assert ref() is None


# ---------------------------------------------------------------- MxA8W4 and FP8 modes

def _mx_args(m=512, k=2048, n=7168, e=8, obs=256, **over):
    """MxA8W4 (Atlas 350 MxA8W4 notes): FP8 x1, FP4 x2 (e,n,k/2 bytes),
    E8M0 block scales (m,k/64,2) and (e,n,k/64,2), transpose_x2 = 1."""
    a = _args(m=m, k=k, n=n, e=e, obs=obs)
    a.x1 = _fake(B.DT_FLOAT8_E4M3FN, m, k)
    a.x2 = _fake(B.DT_FLOAT4_E2M1X2, e, n, k // 2)
    a.scale = _fake(B.DT_FLOAT8_E8M0, e, n, k // 64, 2)
    a.pertoken_scale = _fake(B.DT_FLOAT8_E8M0, m, k // 64, 2)
    a.transpose_x2 = 1
    for key, v in over.items():
        setattr(a, key, v)
    return a


def _fp8_args(m=512, k=2048, n=7168, e=8, obs=256, **over):
    """FP8 E4M3 x1 and x2 (e,n,k), per-channel scale, per-token pertokenScale."""
    a = _args(m=m, k=k, n=n, e=e, obs=obs)
    a.x1 = _fake(B.DT_FLOAT8_E4M3FN, m, k)
    a.x2 = _fake(B.DT_FLOAT8_E4M3FN, e, n, k)
    a.transpose_x2 = 1
    for key, v in over.items():
        setattr(a, key, v)
    return a


MX_CASES = [
    ("mx_ok", _mx_args, {}, B.OK),
    ("mx_no_pertoken", _mx_args, dict(pertoken_scale=B.Tensor()), B.ERR_NULLPTR),
    ("mx_no_scale", _mx_args, dict(scale=B.Tensor()), B.ERR_NULLPTR),
    ("mx_pertoken_fp32", _mx_args, dict(pertoken_scale=_fake(B.DT_FLOAT32, 512, 32, 2)), B.ERR_DTYPE),
    ("mx_per_tensor_pertoken", _mx_args, dict(pertoken_scale=_fake(B.DT_FLOAT8_E8M0, 1)), B.ERR_SHAPE),
    ("mx_row_index_i32", _mx_args, dict(row_index=_fake(B.DT_INT32, 512)), B.ERR_DTYPE),
    ("mx_untransposed", _mx_args, dict(transpose_x2=0), B.ERR_ATTR),
    ("mx_acc_dump", _mx_args, dict(acc_out=_fake(B.DT_INT32, 512, 7168)), B.ERR_UNSUPPORTED),
    # k a multiple of 32 (Atlas 350 MxA8W4 notes), scales (.., ceil(k/64), 2)
    ("mx_k_mult_64_not_128", _mx_args, dict(x1=_fake(B.DT_FLOAT8_E4M3FN, 512, 2112),
                                            x2=_fake(B.DT_FLOAT4_E2M1X2, 8, 7168, 1056),
                                            scale=_fake(B.DT_FLOAT8_E8M0, 8, 7168, 33, 2),
                                            pertoken_scale=_fake(B.DT_FLOAT8_E8M0, 512, 33, 2)), B.OK),
    ("mx_k_mult_32", _mx_args, dict(x1=_fake(B.DT_FLOAT8_E4M3FN, 512, 96), x2=_fake(B.DT_FLOAT4_E2M1X2, 8, 7168, 48),
                                    scale=_fake(B.DT_FLOAT8_E8M0, 8, 7168, 2, 2),
                                    pertoken_scale=_fake(B.DT_FLOAT8_E8M0, 512, 2, 2)), B.OK),
    ("mx_k_mult_32_floor_scales", _mx_args, dict(x1=_fake(B.DT_FLOAT8_E4M3FN, 512, 96),
                                                 x2=_fake(B.DT_FLOAT4_E2M1X2, 8, 7168, 48),
                                                 scale=_fake(B.DT_FLOAT8_E8M0, 8, 7168, 1, 2),
                                                 pertoken_scale=_fake(B.DT_FLOAT8_E8M0, 512, 1, 2)), B.ERR_SHAPE),
    ("mx_k_not_mult_32", _mx_args, dict(x1=_fake(B.DT_FLOAT8_E4M3FN, 512, 80), x2=_fake(B.DT_FLOAT4_E2M1X2, 8, 7168, 40),
                                        scale=_fake(B.DT_FLOAT8_E8M0, 8, 7168, 2, 2),
                                        pertoken_scale=_fake(B.DT_FLOAT8_E8M0, 512, 2, 2)), B.ERR_SHAPE),
    ("mx_scale_shape", _mx_args, dict(scale=_fake(B.DT_FLOAT8_E8M0, 8, 7168, 64)), B.ERR_SHAPE),
    ("fp8_ok", _fp8_args, {}, B.OK),
    ("fp8_per_tensor_pertoken", _fp8_args, dict(pertoken_scale=_fake(B.DT_FLOAT32, 1)), B.OK),
    ("fp8_pertoken_len", _fp8_args, dict(pertoken_scale=_fake(B.DT_FLOAT32, 2)), B.ERR_SHAPE),
    ("fp8_bf16_scale", _fp8_args, dict(scale=_fake(B.DT_BFLOAT16, 8, 1, 7168)), B.OK),
    ("fp8_untransposed", _fp8_args, dict(transpose_x2=0, x2=_fake(B.DT_FLOAT8_E4M3FN, 8, 2048, 7168)), B.OK),
    ("fp8_untransposed_k_mismatch", _fp8_args, dict(transpose_x2=0, x2=_fake(B.DT_FLOAT8_E4M3FN, 8, 7168, 2048)),
     B.ERR_SHAPE),
    ("fp8_transpose_value", _fp8_args, dict(transpose_x2=2), B.ERR_ATTR),
    ("fp8_row_index_i32", _fp8_args, dict(row_index=_fake(B.DT_INT32, 512)), B.ERR_DTYPE),
    ("fp8_acc_dump", _fp8_args, dict(acc_out=_fake(B.DT_INT32, 512, 7168)), B.ERR_UNSUPPORTED),
    ("fp8_x2_int8", _fp8_args, dict(x2=_fake(B.DT_INT8, 8, 7168, 2048)), B.ERR_DTYPE),
]


@pytest.mark.parametrize("name,make,over,code", MX_CASES, ids=[c[0] for c in MX_CASES])
def test_mx_and_fp8_stage_one(name, make, over, code):
    st, _ = _ws(make(**over))
    assert st == code, (B.STATUS_NAMES.get(st), B.STATUS_NAMES.get(code))


# ---------------------------------------------------------------- producer step (quantise + permute)

def _qp_args(T=512, k=2048, K=8, e=32, **over):
    a = B.QpArgs()
    a.hidden = _fake(B.DT_BFLOAT16, T, k)
    a.expert_ids = _fake(B.DT_INT64, T, K)
    a.topk_weights = _fake(B.DT_FLOAT32, T, K)
    a.x1 = _fake(B.DT_INT8, T * K, k)
    a.pertoken_scale = _fake(B.DT_FLOAT32, T * K)
    a.logit = _fake(B.DT_FLOAT32, T * K)
    a.row_index = _fake(B.DT_INT64, T * K)
    a.group_list = _fake(B.DT_INT64, e)
    a.group_list_type = 1
    for key, v in over.items():
        setattr(a, key, v)
    return a


def _qp_ws(a):
    n = ctypes.c_size_t(12345)
    st = B.lib().gmm_quant_permute_workspace(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


def test_quant_permute_workspace_formula():
    """Three int32 sections: one per (expert, chunk of 256 entries), one per
    expert, one per entry."""
    st, ws = _qp_ws(_qp_args(T=512, K=8, e=32))
    nchunks = (512 * 8 + 255) // 256
    r = lambda v: (v + 255) // 256 * 256
    assert st == B.OK and ws == r(32 * nchunks * 4) + r(32 * 4) + r(512 * 8 * 4)
    assert _qp_ws(_qp_args(T=0, K=8, e=4, x1=_fake(B.DT_INT8, 0, 2048))) == (B.OK, 256)


QP_CASES = [
    ("ok_int32_ids_rows", dict(expert_ids=_fake(B.DT_INT32, 512, 8), row_index=_fake(B.DT_INT32, 4096)), B.OK),
    ("ok_no_weights", dict(topk_weights=B.Tensor(), logit=B.Tensor()), B.OK),
    ("weights_without_logit", dict(logit=B.Tensor()), B.ERR_NULLPTR),
    ("logit_without_weights", dict(topk_weights=B.Tensor()), B.ERR_NULLPTR),
    ("no_hidden", dict(hidden=B.Tensor()), B.ERR_NULLPTR),
    ("hidden_f32", dict(hidden=_fake(B.DT_FLOAT32, 512, 2048)), B.ERR_DTYPE),
    ("ids_f32", dict(expert_ids=_fake(B.DT_FLOAT32, 512, 8)), B.ERR_DTYPE),
    ("x1_fp8_per_token", dict(x1=_fake(B.DT_FLOAT8_E4M3FN, 4096, 2048)), B.OK),
    ("x1_fp8_mx", dict(x1=_fake(B.DT_FLOAT8_E4M3FN, 4096, 2048),
                       pertoken_scale=_fake(B.DT_FLOAT8_E8M0, 4096, 32, 2)), B.OK),
    ("x1_fp8_mx_scale_shape", dict(x1=_fake(B.DT_FLOAT8_E4M3FN, 4096, 2048),
                                   pertoken_scale=_fake(B.DT_FLOAT8_E8M0, 4096, 64)), B.ERR_SHAPE),
    ("x1_int8_e8m0_scale", dict(pertoken_scale=_fake(B.DT_FLOAT8_E8M0, 4096, 32, 2)), B.ERR_DTYPE),
    ("x1_fp4", dict(x1=_fake(B.DT_FLOAT4_E2M1X2, 4096, 1024)), B.ERR_DTYPE),
    ("group_list_i32", dict(group_list=_fake(B.DT_INT32, 32)), B.ERR_DTYPE),
    ("group_list_type", dict(group_list_type=2), B.ERR_ATTR),
    ("k_not_mult_16", dict(hidden=_fake(B.DT_BFLOAT16, 512, 2040), x1=_fake(B.DT_INT8, 4096, 2040)), B.ERR_SHAPE),
    ("top_k_65", dict(expert_ids=_fake(B.DT_INT64, 512, 65), topk_weights=_fake(B.DT_FLOAT32, 512, 65)),
     B.ERR_SHAPE),
    ("ids_rows", dict(expert_ids=_fake(B.DT_INT64, 511, 8)), B.ERR_SHAPE),
    ("x1_rows", dict(x1=_fake(B.DT_INT8, 4095, 2048)), B.ERR_SHAPE),
    ("pts_len", dict(pertoken_scale=_fake(B.DT_FLOAT32, 512)), B.ERR_SHAPE),
    ("too_many_experts", dict(group_list=_fake(B.DT_INT64, 1025)), B.ERR_SHAPE),
    ("misaligned_x1", dict(x1=_fake(B.DT_INT8, 4096, 2048, ptr=0x7000008)), B.ERR_ALIGN),
]


@pytest.mark.parametrize("name,over,code", QP_CASES, ids=[c[0] for c in QP_CASES])
def test_quant_permute_stage_one(name, over, code):
    st, ws = _qp_ws(_qp_args(**over))
    assert st == code, (B.STATUS_NAMES.get(st), B.STATUS_NAMES.get(code))
    if code != B.OK:
        assert ws == 12345


# ---------------------------------------------------------------- no fallback, bench contract

def test_binding_fails_loudly_without_the_library(monkeypatch):
    """The product path has no CPU fallback: without the built library every
    entry point raises."""
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libgmmfr.so"))
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()
    with pytest.raises(RuntimeError, match="missing"):
        B.workspace_size(_args())


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with a message."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


# ---------------------------------------------------------------- allocation-free entry point

def test_noalloc_rejects_plans_larger_than_its_scratch_before_device_work():
    """The allocation-free entry point validates and sizes on the host and
    rejects a plan whose workspace exceeds its fixed scratch array (here the
    ordered combine's m*n*4 bytes of contributions) before touching a device,
    so this runs without one; validation errors come first."""
    a = _args(m=8192, n=7168, obs=1024, e=8)  # fake pointers, never dereferenced
    a.combine = B.COMBINE["ordered"]
    assert 8192 * 7168 * 4 > B.NOALLOC_SCRATCH_BYTES
    assert B.lib().gmm_finalize_routing_noalloc(ctypes.byref(a), None) == B.ERR_WORKSPACE
    a.deterministic = 1
    a.combine = B.COMBINE["auto"]
    assert B.lib().gmm_finalize_routing_noalloc(ctypes.byref(a), None) == B.ERR_WORKSPACE
    a.x1 = B.Tensor()
    assert B.lib().gmm_finalize_routing_noalloc(ctypes.byref(a), None) == B.ERR_NULLPTR
    assert B.lib().gmm_finalize_routing_noalloc(None, None) == B.ERR_NULLPTR


def test_row_lookup_hint_is_checked():
    """tuningConfig[3] picks the ordered combine's row lookup: 0, 1 or 2."""
    a = _args(m=4096, n=7168, obs=512, e=8)
    info = B.PlanInfo()
    for v, want in ((0, B.OK), (1, B.OK), (2, B.OK), (3, B.ERR_ATTR), (-1, B.ERR_ATTR)):
        hint = (ctypes.c_int64 * 4)(0, 0, 0, v)
        a.tuning_config = ctypes.cast(hint, ctypes.POINTER(ctypes.c_int64))
        a.tuning_config_len = 4
        assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == want


@pytest.mark.parametrize("maker,m,e,hint,want_m,want_name", [
    (_fp8_args, 131072, 32, 0, 256, "mx_gemm_kernel<256,256,128,4x2,s2,fp8xfp8>"),  # large experts: eight waves
    (_fp8_args, 4096, 8, 0, 128, "mx_gemm_kernel<128,256,64,2x2,s3,fp8xfp8>"),
    (_mx_args, 131072, 32, 0, 128, "mx_gemm_kernel<128,256,64,2x2,s4,fp8xfp4>"),    # MxA8W4 keeps 128 rows
    (_mx_args, 4096, 8, 256, 256, "mx_gemm_kernel<256,256,64,4x2,s4,fp8xfp4>"),     # unless asked
])
def test_fp8_tile_choice(maker, m, e, hint, want_m, want_name):
    a = maker(m=m, e=e, obs=m // 8)
    if hint:
        tc = (ctypes.c_int64 * 2)(0, hint)
        a.tuning_config = ctypes.cast(tc, ctypes.POINTER(ctypes.c_int64))
        a.tuning_config_len = 2
    info = B.PlanInfo()
    assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.OK
    assert (info.tile_m, info.tile_n) == (want_m, 256)
    assert info.tile_k == (128 if ",s2," in want_name else 64)
    assert info.gemm_kernel.decode() == want_name


def test_fp8_big_tile_takes_128_k_per_stage_when_k_allows():
    for k, want in ((2048, "mx_gemm_kernel<256,256,128,4x2,s2,fp8xfp8>"), (2112, "mx_gemm_kernel<256,256,64,4x2,s3,fp8xfp8>")):
        a = _fp8_args(m=131072, k=k, e=32, obs=16384, x1=_fake(B.DT_FLOAT8_E4M3FN, 131072, k),
                      x2=_fake(B.DT_FLOAT8_E4M3FN, 32, 7168, k))
        info = B.PlanInfo()
        assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.OK
        assert info.gemm_kernel.decode() == want


@pytest.mark.parametrize("k,want", [
    (2048, "gmm_kernel<128,256,128,2x2,s2,i4,cont>"),   # 128 k per stage, two stages
    (128, "gmm_kernel<128,256,128,2x2,s2,i4>"),         # one k-step: tile by tile
    (2112, "gmm_kernel<128,256,64,2x2,s3,i4,cont>"),    # k % 128 != 0: 64 k, three stages
])
def test_int4_128_row_tile_stage_depth(k, want):
    a = _args(m=32768, k=k, e=64, obs=4096, int4=True)
    info = B.PlanInfo()
    assert B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info)) == B.OK
    assert info.gemm_kernel.decode() == want
    assert info.tile_k == (128 if ",s2," in want else 64)


def _plan_with(a, tc):
    hint = (ctypes.c_int64 * len(tc))(*tc)
    a.tuning_config = ctypes.cast(hint, ctypes.POINTER(ctypes.c_int64))
    a.tuning_config_len = len(tc)
    info = B.PlanInfo()
    st = B.lib().gmm_finalize_routing_plan(ctypes.byref(a), ctypes.byref(info))
    return st, info


def test_hybrid_request_is_checked():
    """tuningConfig[4]: 0 .. 7 atomic column tiles in every 8; other values ATTR."""
    a = _args(m=4096, n=7168, obs=512, e=8)
    for v, want in ((0, B.OK), (1, B.OK), (7, B.OK), (8, B.ERR_ATTR), (-1, B.ERR_ATTR)):
        assert _plan_with(a, [0, 0, 0, 0, v])[0] == want


@pytest.mark.parametrize("m,k,e,int4,tile", [
    (4096, 2048, 8, False, 0),      # 128-row tile, 64 k in three stages
    (131072, 2048, 32, False, 0),   # 256-row tile, 128 k in two stages
    (32768, 2048, 64, True, 0),     # int4 weights, 128-row tile with 128 k per stage
    (4096, 192, 8, False, 128),     # three k-steps: the continuous pipeline's minimum
])
def test_hybrid_plan_where_available(m, k, e, int4, tile):
    a = _args(m=m, k=k, e=e, obs=m // 8, int4=int4)
    st, ordered = _plan_with(a, [0, tile])
    assert st == B.OK
    st, info = _plan_with(a, [0, tile, 0, 0, 3])
    assert st == B.OK
    assert info.combine == B.COMBINE_HYBRID and info.hybrid_atomic == 3
    assert info.gemm_kernel.decode() == ordered.gemm_kernel.decode()
    a.deterministic = 1  # the ordered combine's workspace
    a.tuning_config_len = 0
    assert _ws(a)[1] == info.workspace_bytes


@pytest.mark.parametrize("case", ["deterministic", "atomic", "ordered", "short_k", "k64_stages", "fp8", "mx", "tile32"])
def test_hybrid_request_ignored_elsewhere(case):
    kw = dict(m=4096, k=2048, e=8, obs=512)
    if case == "short_k":
        kw["k"] = 128          # one k-step: tile by tile
    if case == "k64_stages":
        kw.update(m=131072, e=32, obs=16384, k=2112)  # the 256-row tile with 64 k in four stages
    if case == "fp8":
        a = _fp8_args(m=4096, e=8, obs=512)
    elif case == "mx":
        a = _mx_args(m=4096, e=8, obs=512)
    else:
        a = _args(**kw)
    if case == "deterministic":
        a.deterministic = 1
    if case in ("atomic", "ordered"):
        a.combine = B.COMBINE[case]
    st, info = _plan_with(a, [0, 32 if case == "tile32" else 0, 0, 0, 3])
    assert st == B.OK
    assert info.combine != B.COMBINE_HYBRID and info.hybrid_atomic == 0
