"""Helpers for GPU tests: move a Problem to the device and call the library."""
import numpy as np

from quantized_moe_grouped_amd import binding as B

ATOMIC_RTOL = 1e-5   # max|gpu - ref| <= 1e-5 * max|ref| in the unordered mode


def to_device(p, dev="cuda"):
    import torch

    def T(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def bf16(a):
        return None if a is None else T(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)

    if getattr(p, "mx", False):
        return {
            "x1": T(p.x1).view(torch.float8_e4m3fn),
            "x2": T(p.x2).view(torch.float4_e2m1fn_x2),
            "scale": T(p.scale).view(torch.float8_e8m0fnu),
            "pertoken_scale": T(p.pertoken_scale).view(torch.float8_e8m0fnu),
            "logit": T(p.logit),
            "group_list": T(p.group_list),
            "row_index": T(p.row_index),
            "shared_input": bf16(p.shared_input),
        }
    if getattr(p, "fp8", False):
        return {
            "x1": T(p.x1).view(torch.float8_e4m3fn),
            "x2": T(p.x2).view(torch.float8_e4m3fn),
            "scale": None if p.scale is None else (bf16(p.scale) if p.scale_bf16 else T(p.scale)),
            "pertoken_scale": T(p.pertoken_scale),
            "logit": T(p.logit),
            "group_list": T(p.group_list),
            "row_index": T(p.row_index),
            "shared_input": bf16(p.shared_input),
        }
    return {
        "x1": T(p.x1),
        "x2": T(p.x2),
        "scale": None if p.scale is None else (bf16(p.scale) if p.scale_bf16 else T(p.scale)),
        "pertoken_scale": T(p.pertoken_scale),
        "logit": T(p.logit),
        "group_list": T(p.group_list),
        "row_index": T(p.row_index),
        "shared_input": bf16(p.shared_input),
    }


def call(p, d, out, *, deterministic=False, combine="auto", acc=None, tuning_config=None, workspace=None):
    B.gmm_finalize_routing(
        d["x1"], d["x2"], d["group_list"], out,
        scale=d["scale"], pertoken_scale=d["pertoken_scale"], logit=d["logit"], row_index=d["row_index"],
        shared_input=d["shared_input"], shared_input_offset=p.shared_input_offset if p.shared_input is not None else 0,
        group_list_type=p.group_list_type, deterministic=deterministic, combine=combine, acc_out=acc,
        tuning_config=tuning_config, workspace=workspace, transpose_x2=getattr(p, "x2_transposed", False))


def plan_of(p, d, *, deterministic=False, combine="auto", tuning_config=None):
    """The plan the library takes for these arguments (host only)."""
    import torch
    out = torch.empty((p.output_bs, p.n), dtype=torch.float32, device="cuda")
    args, keep = B.make_args(
        d["x1"], d["x2"], d["group_list"], out,
        scale=d["scale"], pertoken_scale=d["pertoken_scale"], logit=d["logit"], row_index=d["row_index"],
        shared_input=d["shared_input"], shared_input_offset=p.shared_input_offset if p.shared_input is not None else 0,
        group_list_type=p.group_list_type, deterministic=deterministic, combine=combine,
        tuning_config=tuning_config, transpose_x2=getattr(p, "x2_transposed", False))
    plan = B.plan(args)
    del keep
    return plan


def hybrid_ordered_columns(n, atomic_tiles):
    """Columns the hybrid combine folds through the ordered reduce: those of
    the 256-column tiles nt with nt % 8 >= atomic_tiles."""
    return (np.arange(n) // 256) % 8 >= atomic_tiles


def assert_hybrid(got, ref, atomic_tiles):
    """Hybrid combine: every element within the unordered tolerance, and the
    columns of the ordered tiles bit-exact."""
    got = np.asarray(got, dtype=np.float32)
    assert_close_atomic(got, ref)
    cols = hybrid_ordered_columns(got.shape[1], atomic_tiles)
    assert_bitexact(got[:, cols], np.asarray(ref, dtype=np.float32)[:, cols])


def run_gpu(p, d=None, *, deterministic=False, combine="auto", want_acc=False, tuning_config=None,
            acc_sentinel=-0x55555556):
    import torch
    if d is None:
        d = to_device(p)
    out = torch.full((p.output_bs, p.n), float("nan"), dtype=torch.float32, device="cuda")
    acc = None
    if want_acc:
        acc = torch.full((p.m, p.n), acc_sentinel, dtype=torch.int32, device="cuda")
    call(p, d, out, deterministic=deterministic, combine=combine, acc=acc, tuning_config=tuning_config)
    torch.cuda.synchronize()
    return out, acc


def assert_close_atomic(got, ref):
    ref = np.asarray(ref, dtype=np.float32)
    got = np.asarray(got, dtype=np.float32)
    assert np.isfinite(got).all()
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(got.astype(np.float64) - ref.astype(np.float64)).max()) if ref.size else 0.0
    assert err <= ATOMIC_RTOL * scale, f"max err {err} > {ATOMIC_RTOL} * {scale}"


def assert_bitexact(got, ref):
    got = np.asarray(got, dtype=np.float32)
    ref = np.asarray(ref, dtype=np.float32)
    bad = ~((got == ref) | (np.isnan(got) & np.isnan(ref)))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{int(bad.sum())} mismatches, first {idx.tolist()}: "
                             f"{[(float(got[tuple(i)]), float(ref[tuple(i)])) for i in idx]}")


def covered_mask(p):
    import oracle
    s, e = oracle.group_ranges(p)
    mask = np.zeros(p.m, dtype=bool)
    for a, b in zip(s, e):
        mask[a:b] = True
    return mask
